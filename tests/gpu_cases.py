"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the float64 oracle on the same seeded inputs.

The tolerance metric is the oracle-normalised max error,
``max|O_gpu - O_ref| / max|O_ref|``, over the rows compared (the inputs are
N(0,1)/8, so raw outputs are ~1e-3 and a raw max-abs bound would pass an
all-zero output).  Bounds: 2e-3 for FP16, 2e-2 for FP8.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from oracle import icl

TOL = {B.SDM_ICL_PREC_FP16: 2e-3, B.SDM_ICL_PREC_FP8_E4M3: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def norm_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = got.astype(np.float64)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / scale if scale > 0 else float(np.max(np.abs(got)))


class Run:
    """Device copies of one workload plus the oracle's cache."""

    def __init__(self, w: gen.Workload, oracle_codes: bool = True):
        self.w = w
        self.x = gen.make_inputs(w)
        x = self.x
        self.q = to_dev(x.q_ctx)
        self.k = to_dev(x.k_ctx)
        self.v = to_dev(x.v_ctx)
        self.gate = to_dev(x.gate_ctx) if w.scale_mode == gen.SCALE_GATED_LOG else None
        self.coef = x.head_coef if w.scale_mode != gen.SCALE_NONE else None
        self.qq = to_dev(x.q_query)
        self.gq = to_dev(x.gate_query) if w.scale_mode == gen.SCALE_GATED_LOG else None
        self._oracle = None
        self._oracle_codes = oracle_codes

    @property
    def oracle(self) -> icl.OracleCache:
        if self._oracle is None:
            x, w = self.x, self.w
            self._oracle = icl.fit(x.q_ctx, x.k_ctx, x.v_ctx, w.length_list(), w.scale_mode, w.precision,
                                   self.coef, x.gate_ctx if self.gate is not None else None,
                                   keep_codes=self._oracle_codes)
        return self._oracle

    def fit(self, out_ctx: bool):
        import torch
        out = torch.empty_like(self.q) if out_ctx else None
        if out is not None:
            out.fill_(float("nan"))
        cache = B.sdm_icl_attn_fit(self.q, self.k, self.v, self.w.length_list(), self.w.scale_mode,
                                   self.w.precision, self.coef, self.gate, out)
        return cache, out

    def query(self, cache, rows=None):
        q = self.qq if rows is None else self.qq[:, rows[0]:rows[1]].contiguous()
        g = None
        if self.gq is not None:
            g = self.gq if rows is None else self.gq[:, rows[0]:rows[1]].contiguous()
        return B.sdm_icl_attn_query(cache, q, g)

    def ref_context(self, rows, heads=None, b: int = 0) -> np.ndarray:
        gate = self.x.gate_ctx if self.gate is not None else None
        return parallel_rows(lambda r, h: icl.context_outputs(self.oracle, self.x.q_ctx, gate, r, b=b,
                                                               heads=h),
                             rows, self.w.heads if heads is None else heads)

    def ref_query(self, rows, heads=None, b: int = 0) -> np.ndarray:
        rows = np.asarray(rows)
        gate_all = self.x.gate_query[b] if self.gq is not None else None

        def one(r, h):
            g = None if gate_all is None else gate_all[r]
            return icl.attend(self.oracle, self.x.q_query[b, r], g, b=b, heads=h)
        return parallel_rows(one, rows, self.w.heads if heads is None else heads)


def parallel_rows(fn, rows, heads) -> np.ndarray:
    """Evaluate the oracle over (row block, head) pieces in a thread pool.

    ``fn(rows, [h])`` is an oracle call that returns float64 ``[len(rows), H,
    D]`` with head h filled.  Each piece is the oracle's own computation on a
    subset (rows and heads are independent in attention), so the result is
    the same as one call; numpy releases the GIL inside its array operations,
    so the pieces run on the host's cores.  BLAS is held to one thread per
    piece; each piece is one head and a share of the rows, so that it decodes
    that head's keys once.
    """
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(heads) if not isinstance(heads, int) else list(range(heads))
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    groups = max(1, -(-workers // len(heads)))
    block = max(1, -(-rows.size // groups))
    pieces = [(r0, h) for h in heads for r0 in range(0, rows.size, block)]
    parts = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None

    def run(piece):
        r0, h = piece
        parts[piece] = fn(rows[r0:r0 + block], [h])

    workers = min(workers, len(pieces))
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=workers) as pool:
                list(pool.map(run, pieces))
    else:  # pragma: no cover
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(run, pieces))
    out = None
    for (r0, h), part in parts.items():
        if out is None:
            out = np.zeros((rows.size,) + part.shape[1:], dtype=np.float64)
        out[r0:r0 + block, h] = part[:, h]
    if out is None:
        out = np.zeros((0, 0, 0))
    return out
