"""The method, written out plainly in float64 (test infrastructure only).

Sources (page titles as printed on the pages):

* "Fuse shared-length query scaling during inference" -- Problem identified:
  the LogScale factor of a head is its coefficient times the log of the key
  length all rows share; the gated variant also takes tanh of a gate, adds
  one and multiplies, each as its own eager step.  Solution: the length is
  handled in float32 and each intermediate keeps the dtype rounding the
  eager code gives it.  Summary (sequence diagram): the log is clamped.
* "[FP8 3/4] Integrate FP8 attention and caching into TabICLv2" -- intro:
  Q/K/V of intermediate ICL layers are quantised to FP8 above 8,192 unmasked
  context rows; Q scales are derived from the context so cached prediction
  does not depend on how queries are batched; ``model.fit`` builds the cache
  and ``model.predict`` reuses it.  Walkthrough: Q/K/V come from one shared
  projection and the attention itself is PyTorch's scaled dot-product
  attention (softmax scale 1/sqrt(head_dim)).

Readings where the pages are silent (each is a choice, listed with its
reason in the design notes of the repository):

* length: ``L32 = fp32(ln(max(n, 1)))`` (natural log; the clamp makes n <= 1
  give 0); the per-head factor is ``k_h = fp16(fp32(L32 * c_h))``.
* LogScale: ``q~ = fp16(q * k_h)``.  GatedLogScale:
  ``q~ = fp16(fp16(q * k_h) * fp16(1 + fp16(tanh g)))`` with one gate value
  per row and head.
* FP8 scales per (batch, head) from the amax over valid rows, the same rule
  for Q, K and V: ``s = fp32(a / 448)``, ``inv = fp32(448 / a)`` (a = 0
  gives s = inv = 1); codes are ``e4m3(clamp(fp32(x * inv), +-448))`` and
  the dequantised operand is ``code * s``.  Q's amax is taken over the
  *scaled* context queries (what is quantised); query rows reuse the
  context's Q scale and saturate above it, so a query row's result does not
  depend on the other rows of its batch.
* masked context rows (index >= n) are not keys, not part of n and not part
  of any amax; their outputs are zero.
* per-batch lengths (the pages' fused path covers one shared int and falls
  back for tensor lengths): element b behaves as a batch of one with n_b
  rows (its own length scalar, head factors, FP8 scales and keys); AUTO
  precision follows the longest context of the call.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .numerics import E4M3_MAX, E4M3_VALUES, e4m3_encode, e4m3_round

SCALE_NONE, SCALE_LOG, SCALE_GATED_LOG = 0, 1, 2
PREC_FP16, PREC_FP8_E4M3, PREC_AUTO, PREC_SCOPED = 0, 1, 2, 3
FP8_MIN_CONTEXT_ROWS = 8192


# ---------------------------------------------------------------------------
# Shared-length query scaling ("Fuse shared-length query scaling during
# inference": Problem identified, Solution)
# ---------------------------------------------------------------------------

def length_scalar(n: int) -> np.float32:
    """float32 log of the shared key length, clamped so that n <= 1 gives 0."""
    return np.float32(math.log(max(int(n), 1)))


def head_factors(L32: np.float32, head_coef: np.ndarray) -> np.ndarray:
    """Per-head factor in float32 (length x coefficient), then converted to fp16."""
    return (np.float32(L32) * np.asarray(head_coef, dtype=np.float32)).astype(np.float16)


def gate_factor(gate: np.ndarray) -> np.ndarray:
    """fp16(1 + fp16(tanh g)), each pass rounded to fp16 as in eager fp16 code."""
    t = np.tanh(np.asarray(gate, dtype=np.float16).astype(np.float64)).astype(np.float16)
    return (np.float32(1.0) + t.astype(np.float32)).astype(np.float16)


def scale_queries(q: np.ndarray, mode: int, k_h: Optional[np.ndarray],
                  gate: Optional[np.ndarray] = None) -> np.ndarray:
    """Scaled query rows q~ (fp16) for q ``[..., H, D]`` and gate ``[..., H]``.

    NONE leaves q unchanged; LOG multiplies by k_h with one fp16 rounding
    (the product of two fp16 numbers is exact in float32); GATED further
    multiplies by the gate factor with one more fp16 rounding.
    """
    q = np.asarray(q, dtype=np.float16)
    if mode == SCALE_NONE:
        return q.copy()
    kh = np.asarray(k_h, dtype=np.float16).astype(np.float32)[:, None]
    if q.size >= (1 << 20):
        # fp16(q * k_h) depends only on q's 16-bit pattern for a given head:
        # evaluate the same expression once per pattern and index it
        allx = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
        qk = np.empty_like(q)
        bits = q.view(np.uint16)
        for h in range(q.shape[-2]):
            with np.errstate(over="ignore", invalid="ignore"):   # inf/NaN patterns
                table = (allx * kh[h, 0]).astype(np.float16)
            qk[..., h, :] = table[bits[..., h, :]]
    else:
        qk = (q.astype(np.float32) * kh).astype(np.float16)
    if mode == SCALE_LOG:
        return qk
    if mode != SCALE_GATED_LOG:
        raise ValueError(f"unknown scale mode {mode}")
    u = gate_factor(gate).astype(np.float32)[..., None]
    return (qk.astype(np.float32) * u).astype(np.float16)


# ---------------------------------------------------------------------------
# FP8 e4m3 quantisation with per-head, context-derived scales ("[FP8 3/4]
# Integrate FP8 attention and caching into TabICLv2", introduction)
# ---------------------------------------------------------------------------

def select_precision(n: int, requested: int, fp8_scope: bool = False) -> int:
    """Precision of one attention call with n unmasked context rows.

    AUTO: FP8 only above 8,192 unmasked context rows.  SCOPED: the rule of an
    intermediate ICL layer under the opt-in FP8 scope of the TabICLv2 FP8
    page (introduction): FP8 iff the scope enables it *and* n > 8,192, else
    the normal precision; a final layer keeps normal precision by asking for
    FP16.  Explicit FP16 / FP8 are honoured as given.
    """
    if requested == PREC_AUTO:
        return PREC_FP8_E4M3 if n > FP8_MIN_CONTEXT_ROWS else PREC_FP16
    if requested == PREC_SCOPED:
        return PREC_FP8_E4M3 if (fp8_scope and n > FP8_MIN_CONTEXT_ROWS) else PREC_FP16
    return requested


def fp8_scale(amax) -> tuple:
    """(s, inv) in float32 for one tensor's amax: s = a/448, inv = 448/a; a = 0 -> 1."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a / np.float32(E4M3_MAX)), np.float32(np.float32(E4M3_MAX) / a)


def amax_rows(x: np.ndarray) -> np.ndarray:
    """max |x| over rows and head_dim for finite fp16 x ``[rows, H, D]`` -> ``[H]``.

    For finite IEEE numbers, |x| orders exactly as the bit pattern with the
    sign bit cleared, read as an unsigned integer; the maximum is taken on
    those patterns and converted back, so it is exact."""
    mag = np.asarray(x, dtype=np.float16).view(np.uint16) & np.uint16(0x7FFF)
    top = mag.max(axis=2).max(axis=0).astype(np.uint16)
    return top.view(np.float16).astype(np.float64)


def quantize(x: np.ndarray, inv) -> np.ndarray:
    """E4M3 values (float64 on the grid) of fp16 x scaled by the float32 inverse scale."""
    y = np.asarray(x, dtype=np.float16).astype(np.float32) * np.float32(inv)
    y = np.clip(y.astype(np.float32), -E4M3_MAX, E4M3_MAX)
    return e4m3_round(y)


def _code_table(inv) -> np.ndarray:
    """quantize + encode evaluated once on every fp16 bit pattern (finite ones;
    NaN/inf patterns map to 0 and never occur in valid rows)."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ok = np.isfinite(x)
    table = np.zeros(65536, dtype=np.uint8)
    table[ok] = e4m3_encode(quantize(x[ok], inv))
    return table


def quantize_codes(x: np.ndarray, inv) -> np.ndarray:
    """E4M3 bit patterns of :func:`quantize`.  x is fp16 and inv is one
    float32, so the code is a function of x's 16-bit pattern: large inputs
    index a table of that function instead of recomputing it per element."""
    x = np.asarray(x, dtype=np.float16)
    if x.size < 65536:
        return e4m3_encode(quantize(x, inv))
    return _code_table(inv)[x.view(np.uint16)]


# ---------------------------------------------------------------------------
# Attention (SDPA semantics, non-causal): O_i = sum_j softmax_j(tau q_i.k_j) v_j
# ---------------------------------------------------------------------------

def attention_rows(qhat: np.ndarray, khat: np.ndarray, vhat: np.ndarray,
                   tau: float) -> np.ndarray:
    """Exact softmax attention of each query row over all given keys, float64.

    ``qhat [m, D]``, ``khat [n, D]``, ``vhat [n, D]``.  Two passes per row:
    the logits' maximum, then exp-weights normalised by their sum.
    """
    q = np.asarray(qhat, dtype=np.float64)
    k = np.asarray(khat, dtype=np.float64)
    v = np.asarray(vhat, dtype=np.float64)
    z = (q @ k.T) * tau
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p @ v) / p.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# fit / predict, as on the TabICLv2 FP8 page (model.fit builds per-layer
# caches, model.predict reuses them)
# ---------------------------------------------------------------------------

@dataclass
class OracleCache:
    """What ``fit`` keeps per batch element b: its key length n_b, scaling
    factors and K/V operands (valid rows only)."""

    lengths: np.ndarray              # int64 [B]: n_b
    heads: int
    head_dim: int
    scale_mode: int
    precision: int
    L32s: np.ndarray                 # float32 [B]
    k_hs: Optional[np.ndarray]       # fp16 [B, H] or None
    scales: np.ndarray               # float32 [3, B, H]: s_q, s_k, s_v (ones for FP16)
    inv: np.ndarray                  # float32 [3, B, H]
    k16: list                        # per b: fp16 [n_b, H, D]
    v16: list
    k_codes_b: Optional[list]        # per b: uint8 [H, n_b, D] (FP8 only)
    v_codes_b: Optional[list]

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def _shared(self) -> None:
        if np.any(self.lengths != self.lengths[0]):
            raise ValueError("the batch elements have different lengths")

    @property
    def n(self) -> int:
        """The shared length (only when every batch element has the same n)."""
        self._shared()
        return int(self.lengths[0])

    @property
    def L32(self) -> np.float32:
        self._shared()
        return self.L32s[0]

    @property
    def k_h(self) -> Optional[np.ndarray]:
        self._shared()
        return None if self.k_hs is None else self.k_hs[0]

    @property
    def k_codes(self) -> Optional[np.ndarray]:
        """uint8 ``[B, H, n, D]`` (shared length only)."""
        self._shared()
        return None if self.k_codes_b is None else np.stack(self.k_codes_b)

    @property
    def v_codes(self) -> Optional[np.ndarray]:
        self._shared()
        return None if self.v_codes_b is None else np.stack(self.v_codes_b)

    def khat(self, b: int, h: int) -> np.ndarray:
        if self.precision == PREC_FP8_E4M3:
            return E4M3_VALUES[self.k_codes_b[b][h]] * np.float64(self.scales[1, b, h])
        return self.k16[b][:, h, :].astype(np.float64)

    def vhat(self, b: int, h: int) -> np.ndarray:
        if self.precision == PREC_FP8_E4M3:
            return E4M3_VALUES[self.v_codes_b[b][h]] * np.float64(self.scales[2, b, h])
        return self.v16[b][:, h, :].astype(np.float64)

    def qhat(self, qt: np.ndarray, b: int, h: int) -> np.ndarray:
        """Operand used for scaled query rows qt ``[m, H, D]`` (fp16) of head h:
        FP8 quantises with the context's Q scale and dequantises with it."""
        x = qt[:, h, :]
        if self.precision == PREC_FP8_E4M3:
            return quantize(x, self.inv[0, b, h]) * np.float64(self.scales[0, b, h])
        return x.astype(np.float64)


def _lengths(n, B: int, N: int) -> np.ndarray:
    """n as one int64 per batch element: a shared int, or a sequence of B."""
    arr = np.asarray(n, dtype=np.int64).reshape(-1)
    if arr.size == 1:
        arr = np.full(B, arr[0], dtype=np.int64)
    if arr.size != B:
        raise ValueError("lengths must be one int or one per batch element")
    if np.any(arr < 1) or np.any(arr > N):
        raise ValueError("need 1 <= n_b <= N_pad")
    return arr


def fit(q: np.ndarray, k: np.ndarray, v: np.ndarray, n, scale_mode: int,
        precision: int, head_coef: Optional[np.ndarray] = None,
        gate: Optional[np.ndarray] = None, keep_codes: bool = True,
        fp8_scope: bool = False) -> OracleCache:
    """Build the cache from context Q/K/V ``[B, N_pad, H, D]``.

    n: the valid rows, one int shared by all batch elements or one per
    element.  Element b is treated exactly as a batch of one with n_b valid
    rows: its own length scalar and head factors, FP8 scales over its own
    valid rows, its own keys.  AUTO precision is decided once for the call by
    the longest context (FP8 iff max n_b > 8,192).
    """
    B, N, H, D = q.shape
    lengths = _lengths(n, B, N)
    prec = select_precision(int(lengths.max()), precision, fp8_scope)
    L32s = np.array([length_scalar(int(nb)) for nb in lengths], dtype=np.float32)
    k_hs = (np.stack([head_factors(L32s[b], head_coef) for b in range(B)])
            if scale_mode != SCALE_NONE else None)
    scales = np.ones((3, B, H), dtype=np.float32)
    inv = np.ones((3, B, H), dtype=np.float32)
    k_codes = v_codes = None
    if prec == PREC_FP8_E4M3:
        k_codes, v_codes = [], []
        for b in range(B):
            nb = int(lengths[b])
            qt = scale_queries(q[b, :nb], scale_mode, None if k_hs is None else k_hs[b],
                               None if gate is None else gate[b, :nb])
            for t, x in enumerate((qt, k[b, :nb], v[b, :nb])):
                a = amax_rows(x)
                for h in range(H):
                    scales[t, b, h], inv[t, b, h] = fp8_scale(a[h])
            kc = np.empty((H, nb, D), dtype=np.uint8)
            vc = np.empty((H, nb, D), dtype=np.uint8)
            for h in range(H):
                kc[h] = quantize_codes(k[b, :nb, h, :], inv[1, b, h])
                vc[h] = quantize_codes(v[b, :nb, h, :], inv[2, b, h])
            k_codes.append(kc)
            v_codes.append(vc)
    return OracleCache(lengths=lengths, heads=H, head_dim=D, scale_mode=scale_mode, precision=prec,
                       L32s=L32s, k_hs=k_hs, scales=scales, inv=inv,
                       k16=[k[b, :int(lengths[b])] for b in range(B)],
                       v16=[v[b, :int(lengths[b])] for b in range(B)],
                       k_codes_b=k_codes, v_codes_b=v_codes)


def attend(cache: OracleCache, q_rows: np.ndarray, gate_rows: Optional[np.ndarray],
           b: int = 0, heads: Optional[Sequence[int]] = None,
           block: int = 128) -> np.ndarray:
    """Outputs (float64 ``[m, H, D]``) of query rows ``q_rows [m, H, D]`` of batch b.

    Rows are scaled with batch element b's length and the coefficients,
    quantised with b's context-derived Q scale in FP8 mode, and attend to b's
    n_b keys.  Rows are evaluated independently, ``block`` at a time to bound
    memory.
    """
    qt = scale_queries(q_rows, cache.scale_mode, None if cache.k_hs is None else cache.k_hs[b],
                       gate_rows)
    m = q_rows.shape[0]
    out = np.zeros((m, cache.heads, cache.head_dim), dtype=np.float64)
    for h in (range(cache.heads) if heads is None else heads):
        kh, vh = cache.khat(b, h), cache.vhat(b, h)
        qh = cache.qhat(qt, b, h)
        for r0 in range(0, m, block):
            out[r0:r0 + block, h] = attention_rows(qh[r0:r0 + block], kh, vh, cache.tau)
    return out


def context_outputs(cache: OracleCache, q: np.ndarray, gate: Optional[np.ndarray],
                    rows: Sequence[int], b: int = 0, heads=None) -> np.ndarray:
    """Self-attention outputs of batch b's given context rows (rows >= n_b give 0)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, cache.heads, cache.head_dim), dtype=np.float64)
    valid = rows < cache.lengths[b]
    if np.any(valid):
        g = None if gate is None else gate[b, rows[valid]]
        out[valid] = attend(cache, q[b, rows[valid]], g, b=b, heads=heads)
    return out


# ---------------------------------------------------------------------------
# The shared Q/K/V projection, with the query scaling applied to its output
# ("[FP8 3/4] Integrate FP8 attention and caching into TabICLv2", walkthrough:
# one shared projection makes Q, K and V before attention; "Fuse shared-length query
# scaling during inference", Solution: the scaling joins the producer of q
# instead of running as separate passes over it)
# ---------------------------------------------------------------------------

def project_qkv(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], heads: int,
                head_dim: int) -> tuple:
    """fp16 (Q, K, V), each ``[..., H, D]``, of hidden rows x ``[..., E]``.

    w is ``[3 H D, E]`` (a linear layer's weight: the Q rows, then K, then V),
    bias ``[3 H D]`` or None, both fp16.  Each output element is the sum
    x . w_n + b_n taken in float64 (fp16 products are exact in it) and
    rounded once to fp16 (nearest even).
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float16).astype(np.float64)
    y = x64 @ w64.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float16).astype(np.float64)
    y16 = y.astype(np.float16)
    hd = heads * head_dim
    shape = x64.shape[:-1] + (heads, head_dim)
    return (y16[..., :hd].reshape(shape), y16[..., hd:2 * hd].reshape(shape),
            y16[..., 2 * hd:].reshape(shape))


def project_scaled(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], heads: int,
                   head_dim: int, mode: int, k_h: Optional[np.ndarray],
                   gate: Optional[np.ndarray] = None) -> tuple:
    """(q~, K, V): the projection with LogScale / GatedLogScale applied to its
    fp16 Q output, exactly as the separate scaling pass would."""
    q, k, v = project_qkv(x, w, bias, heads, head_dim)
    return scale_queries(q, mode, k_h, gate), k, v
