"""Seeded synthetic inputs for row-wise ICL attention.

This module only draws random numbers and rounds them to the storage dtype
(fp16); it holds none of the attention, scaling or quantisation arithmetic.
Both the float64 oracle and the GPU path take their inputs from here.

The recipe follows the workloads of the FP8 TabICLv2 and KumoTabular pages
("[FP8 3/4] Integrate FP8 attention and caching into TabICLv2", results table;
"Stack 4/5", results table): 16K-512K context rows, 1,024 query rows, an ICL
width of 8 heads x 64.  Values are N(0,1)/8 in fp16; the FP8 workloads add
0.1% outliers at +-20 sigma; a padded context tail is filled with NaN so that
any read of a masked row shows up in the output.

Streams (fixed, per config seed): context Q, K, V ``[B, N_pad, H, D]`` and
query Q ``[B, R, H, D]`` come from per-64K-row-chunk generators keyed by
(seed, tensor index 0..3, batch, chunk); from ``default_rng(seed)``, in order:
head coefficients ``[H]`` ~ U(0.5, 1.5) (float32), context gate
``[B, N_pad, H]`` and query gate ``[B, R, H]`` ~ N(0, 1) (fp16), then, if
outliers are on, an outlier count, positions and signs per tensor in the order
context Q, K, V, query Q.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

SCALE_NONE = 0
SCALE_LOG = 1
SCALE_GATED_LOG = 2

PREC_FP16 = 0
PREC_FP8_E4M3 = 1
PREC_AUTO = 2

_CHUNK_ROWS = 65536


@dataclass(frozen=True)
class Workload:
    """One synthetic ICL attention workload.

    ``n_pad`` context rows are allocated, of which the first ``n_valid`` are
    real; rows ``n_valid..n_pad-1`` are masked (NaN-filled when ``nan_tail``).
    ``n_query`` query rows attend to the context.  ``query_batches`` lists the
    query-batch sizes a cached prediction is split into.
    """

    name: str
    seed: int
    n_pad: int
    n_valid: int
    n_query: int
    heads: int = 8
    head_dim: int = 64
    batch: int = 1
    scale_mode: int = SCALE_NONE
    precision: int = PREC_FP16
    outliers: bool = False
    nan_tail: bool = False
    query_batches: tuple = ()
    description: str = ""
    lengths: tuple = ()          # per-batch valid rows (empty: every element has n_valid)

    def valid_rows(self, b: int) -> int:
        """Valid context rows of batch element b."""
        return int(self.lengths[b]) if self.lengths else self.n_valid

    def length_list(self) -> list:
        return [self.valid_rows(b) for b in range(self.batch)]


# The five workloads: tiny FP16, 16K LogScale/GatedLogScale FP16, 128K FP8,
# a 512K cached FP8 prediction and a full 512K FP8 model call with a ragged
# (masked) context tail; and a ragged pair of 128K/64K FP8 contexts in one
# launch (per-batch lengths).
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp16": Workload(
        name="tiny_fp16", seed=0, n_pad=1024, n_valid=1024, n_query=64, heads=4,
        description="1,024 context rows + 64 queries, 4 heads, FP16, no scaling"),
    "ctx16k_log_fp16": Workload(
        name="ctx16k_log_fp16", seed=1, n_pad=16384, n_valid=16384, n_query=1024,
        scale_mode=SCALE_LOG,
        description="16,384 context rows + 1,024 queries, 8 heads, FP16, LogScale"),
    "ctx16k_gated_fp16": Workload(
        name="ctx16k_gated_fp16", seed=1, n_pad=16384, n_valid=16384, n_query=1024,
        scale_mode=SCALE_GATED_LOG,
        description="16,384 context rows + 1,024 queries, 8 heads, FP16, GatedLogScale"),
    "ctx128k_fp8": Workload(
        name="ctx128k_fp8", seed=2, n_pad=131072, n_valid=131072, n_query=1024,
        precision=PREC_FP8_E4M3, outliers=True,
        description="131,072 context rows + 1,024 queries, 8 heads, FP8 e4m3, outliers"),
    "cached512k_fp8_gated": Workload(
        name="cached512k_fp8_gated", seed=3, n_pad=524288, n_valid=524288, n_query=1024,
        scale_mode=SCALE_GATED_LOG, precision=PREC_FP8_E4M3, outliers=True,
        query_batches=(128, 1024),
        description="1,024 GatedLogScale queries against a resident 524,288-row FP8 cache"),
    "ragged128k_fp8": Workload(
        name="ragged128k_fp8", seed=5, batch=2, n_pad=131072, n_valid=131072, n_query=1024,
        precision=PREC_FP8_E4M3, outliers=True, nan_tail=True, lengths=(131072, 65537),
        description="two contexts of 131,072 and 65,537 rows in one launch (rows past each "
                    "length masked) + 1,024 queries per element, FP8 e4m3"),
    "model512k_fp8_log": Workload(
        name="model512k_fp8_log", seed=4, n_pad=524288, n_valid=523288, n_query=1024,
        scale_mode=SCALE_LOG, precision=PREC_FP8_E4M3, outliers=True, nan_tail=True,
        description="524,288 padded context rows (last 1,000 masked) + 1,024 queries, "
                    "FP8 e4m3, LogScale"),
}


def scaled_down(w: Workload, n_pad: int, n_valid: Optional[int] = None,
                n_query: Optional[int] = None, name: Optional[str] = None) -> Workload:
    """The same recipe (seed, modes, distributions) at a smaller size."""
    if n_valid is None:
        tail = w.n_pad - w.n_valid
        n_valid = n_pad - tail if tail < n_pad else n_pad
    return replace(w, name=name or f"{w.name}@{n_pad}", n_pad=n_pad, n_valid=n_valid,
                   n_query=w.n_query if n_query is None else n_query)


def _normal_fp16(seed: int, tensor: int, shape) -> np.ndarray:
    """N(0,1)/8 drawn as float32 and rounded (nearest-even) to fp16.

    Each 64K-row chunk has its own generator, seeded from (seed, tensor,
    batch, chunk) through numpy's SeedSequence, so chunks are drawn in
    parallel threads and the result does not depend on the thread count."""
    out = np.empty(shape, dtype=np.float16)
    rows = shape[1]
    jobs = [(b, r0) for b in range(shape[0]) for r0 in range(0, rows, _CHUNK_ROWS)]

    def fill(job):
        b, r0 = job
        r1 = min(rows, r0 + _CHUNK_ROWS)
        sub = (r1 - r0,) + tuple(shape[2:])
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(seed, spawn_key=(tensor, b, r0 // _CHUNK_ROWS))))
        out[b, r0:r1] = (g.standard_normal(sub, dtype=np.float32) / np.float32(8.0)).astype(np.float16)

    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(fill, jobs))
    return out


def _add_outliers(rng: np.random.Generator, x: np.ndarray) -> None:
    """Set a Binomial(size, 1e-3) number of elements, at uniformly drawn
    positions (with replacement), to +-20 sigma (= +-2.5) with random signs."""
    flat = x.reshape(-1)
    count = int(rng.binomial(flat.size, 1e-3))
    pos = rng.integers(0, flat.size, size=count)
    sign = rng.integers(0, 2, size=count) * 2 - 1
    flat[pos] = (2.5 * sign).astype(np.float16)


@dataclass
class Inputs:
    """Host fp16 arrays of one workload (row-major ``[B, rows, H, D]``)."""

    workload: Workload
    q_ctx: np.ndarray
    k_ctx: np.ndarray
    v_ctx: np.ndarray
    q_query: np.ndarray
    head_coef: np.ndarray
    gate_ctx: np.ndarray
    gate_query: np.ndarray
    extra: dict = field(default_factory=dict)


def make_inputs(w: Workload) -> Inputs:
    """Draw every tensor of workload ``w`` from ``numpy.random.default_rng(w.seed)``."""
    rng = np.random.default_rng(w.seed)
    B, N, H, D, R = w.batch, w.n_pad, w.heads, w.head_dim, w.n_query
    q_ctx = _normal_fp16(w.seed, 0, (B, N, H, D))
    k_ctx = _normal_fp16(w.seed, 1, (B, N, H, D))
    v_ctx = _normal_fp16(w.seed, 2, (B, N, H, D))
    q_query = _normal_fp16(w.seed, 3, (B, R, H, D))
    head_coef = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    gate_ctx = rng.standard_normal((B, N, H), dtype=np.float32).astype(np.float16)
    gate_query = rng.standard_normal((B, R, H), dtype=np.float32).astype(np.float16)
    if w.outliers:
        for t in (q_ctx, k_ctx, v_ctx, q_query):
            _add_outliers(rng, t)
    if w.nan_tail:
        for b in range(B):
            nb = w.valid_rows(b)
            for t in (q_ctx, k_ctx, v_ctx):
                t[b, nb:] = np.float16(np.nan)
            gate_ctx[b, nb:] = np.float16(np.nan)
    return Inputs(w, q_ctx, k_ctx, v_ctx, q_query, head_coef, gate_ctx, gate_query)


def sample_rows(n_valid: int, count: int, seed: int, edge: int = 8) -> np.ndarray:
    """A sorted, seeded subset of ``count`` valid context rows that always
    includes the first and last ``edge`` valid rows."""
    if count >= n_valid:
        return np.arange(n_valid, dtype=np.int64)
    rng = np.random.default_rng(seed + 1000)
    fixed = np.concatenate([np.arange(min(edge, n_valid)),
                            np.arange(max(0, n_valid - edge), n_valid)])
    pool = np.setdiff1d(np.arange(n_valid), fixed)
    pick = rng.choice(pool, size=max(0, count - fixed.size), replace=False)
    return np.unique(np.concatenate([fixed, pick])).astype(np.int64)
