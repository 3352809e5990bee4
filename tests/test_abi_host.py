"""Host-side tests of the C-ABI library (no GPU needed).

The library must load and export every function that include/sdm_icl_attn.h
declares; the host helpers (length scalar, fp16 head factors, precision rule,
split plan) must agree with the oracle; and argument errors must be reported
before anything touches a device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from oracle import icl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm_icl_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_icl_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 13, names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(B._SIGNATURES), "binding and header disagree"
    assert B.sdm_icl_version() == 102


def test_noalloc_query_validates_on_the_host():
    """The no-allocation query rejects an unknown handle before any device
    call (no GPU needed), like the workspace query."""
    lib = B.lib()
    assert lib.sdm_icl_attn_query_noalloc(None, None, None, 4, None, None) == 6
    assert "unknown or released cache" in B.sdm_icl_last_error()
    assert "query_noalloc" in B.sdm_icl_last_error()


@pytest.mark.parametrize("n", [0, 1, 2, 3, 1000, 1024, 8192, 16384, 65537, 131072, 523288, 524288, 10**9])
def test_length_scalar_matches_oracle(n):
    assert B.sdm_icl_length_scalar(n) == icl.length_scalar(n)


def test_head_factors_match_oracle():
    rng = np.random.default_rng(7)
    for n in (1, 2, 1024, 16384, 131072, 523288, 524288):
        for scale in (1.0, 1e-3, 1e-6, 100.0, 5000.0):
            coef = (rng.uniform(0.5, 1.5, 128) * scale).astype(np.float32)
            got = B.sdm_icl_head_factors(n, coef)
            want = icl.head_factors(icl.length_scalar(n), coef)
            np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))
    # ties and overflow at the fp16 edges (L = ln 2 ... via n = 2: L = fp32(ln 2))
    L = float(icl.length_scalar(2))
    edge = np.array([65504.0, 65519.0, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -24,
                     3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11], dtype=np.float64) / L
    coef = edge.astype(np.float32)
    np.testing.assert_array_equal(B.sdm_icl_head_factors(2, coef).view(np.uint16),
                                  icl.head_factors(icl.length_scalar(2), coef).view(np.uint16))


def test_precision_rule_matches_oracle():
    for n in (1, 8191, 8192, 8193, 10**6):
        for req in (0, 1, 2):
            assert B.sdm_icl_select_precision(n, req) == icl.select_precision(n, req)


def test_split_plan_depends_on_n_cus_and_heads_only():
    for n in (1, 63, 64, 65, 1000, 16384, 131072, 523288, 524288):
        for bh in (1, 4, 8, 16, 200):
            s, kps = B.sdm_icl_split_plan(n, 256, bh)
            assert kps % 64 == 0 and s >= 1
            assert (s - 1) * kps < n <= s * kps   # every split holds at least one valid key
            assert kps >= min(256, -(-n // 64) * 64)  # at least 4 tiles unless n is shorter
    # 8 heads on 256 CUs: 96 splits x 8 heads = 3 (split, head) units per CU,
    # 86 key tiles per split
    assert B.sdm_icl_split_plan(524288, 256, 8) == (96, 5504)
    assert B.sdm_icl_split_plan(523288, 256, 8) == (96, 5504)
    assert B.sdm_icl_split_plan(524288, 256, 4) == (191, 2752)
    for bad in ((0, 256, 8), (100, 0, 8), (100, 256, 0)):
        with pytest.raises(B.SdmIclError):
            B.sdm_icl_split_plan(*bad)


def _fit_args(**kw):
    lengths = (ctypes.c_int64 * 1)(100)
    coef = (ctypes.c_float * 8)(*([1.0] * 8))
    base = dict(batch=1, rows_padded=128, heads=8, head_dim=64, lengths=lengths,
                q=0x1000, k=0x2000, v=0x3000, gate=None, head_coef=None, scale_mode=0,
                precision=0, out_ctx=None, stream=None)
    base.update(kw)
    if base.get("head_coef") == "set":
        base["head_coef"] = coef
    return B.FitArgs(**base), (lengths, coef)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1),
    (dict(heads=0), 1),
    (dict(heads=129), 2),
    (dict(head_dim=128), 2),
    (dict(lengths=None), 1),
    (dict(q=None), 1),
    (dict(scale_mode=3), 1),
    (dict(scale_mode=1), 1),                           # LOG without coefficients
    (dict(scale_mode=2, head_coef="set"), 1),          # GATED without gate
    (dict(scale_mode=0, gate=0x4000), 1),              # gate without GATED
    (dict(scale_mode=0, head_coef="set"), 1),          # coefficients without scaling
    (dict(precision=5), 1),
    (dict(rows_padded=50), 1),                         # n = 100 > N_pad
    (dict(q=0x1008), 1),                               # q not 16-byte aligned
    (dict(v=0x3002), 1),
    (dict(out_ctx=0x5004), 1),
    (dict(scale_mode=2, head_coef="set", gate=0x4001), 1),  # odd gate address
])
def test_fit_rejects_bad_arguments_before_any_device_work(kw, status):
    args, keep = _fit_args(**kw)
    h = ctypes.c_void_p()
    st = B.lib().sdm_icl_attn_fit(ctypes.byref(args), ctypes.byref(h))
    assert st == status, B.sdm_icl_last_error()
    assert h.value is None
    assert B.sdm_icl_last_error()


def test_per_batch_lengths_pass_validation_and_bad_ones_are_invalid():
    h = ctypes.c_void_p()
    # differing lengths are valid: the call gets past host validation and
    # stops at the device check (no GPU here) or succeeds on a GPU host
    lengths = (ctypes.c_int64 * 2)(100, 90)
    args, keep = _fit_args(batch=2, lengths=lengths)
    assert B.lib().sdm_icl_attn_fit(ctypes.byref(args), ctypes.byref(h)) not in (1, 2)
    for bad in ((0,), (100, 0), (100, 129)):        # n_b = 0, or n_b > rows_padded = 128
        lengths_bad = (ctypes.c_int64 * len(bad))(*bad)
        args, keep = _fit_args(batch=len(bad), lengths=lengths_bad)
        assert B.lib().sdm_icl_attn_fit(ctypes.byref(args), ctypes.byref(h)) == 1
        assert "lengths[" in B.sdm_icl_last_error()


def test_unknown_handles_are_rejected():
    lib = B.lib()
    bogus = ctypes.c_void_p(0xDEADBEEF)
    size = ctypes.c_size_t()
    assert lib.sdm_icl_attn_query_workspace_size(bogus, 10, ctypes.byref(size)) == 6
    assert lib.sdm_icl_attn_query(bogus, None, None, 0, None, None, 0, None) == 6
    assert lib.sdm_icl_attn_release(bogus) == 6
    assert lib.sdm_icl_attn_release(None) == 6
    info = B.CacheInfo()
    assert lib.sdm_icl_attn_cache_info(bogus, ctypes.byref(info)) == 6


def test_log_scale_validation():
    lib = B.lib()
    coef = (ctypes.c_float * 8)(*([1.0] * 8))
    # GATED without gate, LOG without coef, bad head_dim
    assert lib.sdm_icl_log_scale(0x1000, None, 1, 4, 8, 64, 10, coef, 2, None, 0x2000, None) == 1
    assert lib.sdm_icl_log_scale(0x1000, None, 1, 4, 8, 64, 10, None, 1, None, 0x2000, None) == 1
    assert lib.sdm_icl_log_scale(0x1000, None, 1, 4, 8, 32, 10, coef, 1, None, 0x2000, None) == 2
    # zero rows is a no-op
    assert lib.sdm_icl_log_scale(None, None, 1, 0, 8, 64, 10, coef, 1, None, None, None) == 0


# ----------------------------------------------------------------- FP8 scope (host logic)

def test_scope_stack_nesting_inherit_and_errors():
    lib = B.lib()
    assert B.sdm_icl_scope_fp8() == 0                     # no scope: disabled
    B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_ENABLE)
    try:
        assert B.sdm_icl_scope_fp8() == 1
        B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_INHERIT)
        assert B.sdm_icl_scope_fp8() == 1                 # inherits the enclosing ENABLE
        B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_DISABLE)
        assert B.sdm_icl_scope_fp8() == 0
        B.sdm_icl_scope_pop()
        assert B.sdm_icl_scope_fp8() == 1                 # leaving restores the setting
        B.sdm_icl_scope_pop()
    finally:
        B.sdm_icl_scope_pop()
    assert B.sdm_icl_scope_fp8() == 0
    assert lib.sdm_icl_scope_pop() == 6                   # nothing open
    assert lib.sdm_icl_scope_push(7) == 1                 # unknown setting
    for _ in range(256):
        B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_INHERIT)
    assert lib.sdm_icl_scope_push(B.SDM_ICL_SCOPE_ENABLE) == 6   # depth limit
    for _ in range(256):
        B.sdm_icl_scope_pop()


def test_scope_is_per_thread_in_the_library():
    import threading
    seen = []
    B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_ENABLE)
    try:
        t = threading.Thread(target=lambda: seen.append(B.sdm_icl_scope_fp8()))
        t.start()
        t.join()
    finally:
        B.sdm_icl_scope_pop()
    assert seen == [0]


def test_scoped_precision_matches_oracle():
    for n in (1, 8192, 8193, 10 ** 6):
        assert B.sdm_icl_select_precision(n, B.SDM_ICL_PREC_SCOPED) == \
            icl.select_precision(n, icl.PREC_SCOPED, fp8_scope=False)
        B.sdm_icl_scope_push(B.SDM_ICL_SCOPE_ENABLE)
        try:
            assert B.sdm_icl_select_precision(n, B.SDM_ICL_PREC_SCOPED) == \
                icl.select_precision(n, icl.PREC_SCOPED, fp8_scope=True)
            for req in (0, 1, 2):     # the scope leaves explicit and AUTO precision alone
                assert B.sdm_icl_select_precision(n, req) == icl.select_precision(n, req)
        finally:
            B.sdm_icl_scope_pop()


def test_optimize_is_context_local_and_restores_on_exceptions():
    import asyncio
    import threading
    assert not B.fp8_scope_enabled()
    with B.optimize(attention="fp8"):
        assert B.fp8_scope_enabled()
        with B.optimize(attention=None):
            assert B.fp8_scope_enabled()
        with pytest.raises(KeyError):
            with B.optimize(attention="none"):
                assert not B.fp8_scope_enabled()
                raise KeyError("boom")
        assert B.fp8_scope_enabled()
        other = []
        t = threading.Thread(target=lambda: other.append(B.fp8_scope_enabled()))
        t.start()
        t.join()
        assert other == [False]                           # a new thread starts outside any scope
    assert not B.fp8_scope_enabled()

    async def task(enable, started, out):
        if enable:
            with B.optimize(attention="fp8"):
                started.set()
                await asyncio.sleep(0.01)
                out.append(B.fp8_scope_enabled())
        else:
            await started.wait()
            out.append(B.fp8_scope_enabled())

    async def main():
        started, a, b = asyncio.Event(), [], []
        await asyncio.gather(task(True, started, a), task(False, started, b))
        return a, b

    a, b = asyncio.run(main())
    assert a == [True] and b == [False]                   # tasks do not see each other's scope
    with pytest.raises(ValueError):
        with B.optimize(attention="int4"):
            pass


# ----------------------------------------------------------------- cache import (host validation)

def _import_status(k, v, sc, lengths=(3,), mode=0, prec=1, coef=None):
    args, keep = B.import_args(k, v, sc, list(lengths), mode, prec, coef)
    h = ctypes.c_void_p()
    st = B.lib().sdm_icl_attn_cache_import(ctypes.byref(args), ctypes.byref(h))
    return st


def test_import_validates_before_touching_the_device():
    k = np.zeros((1, 2, 3, 64), dtype=np.uint8)
    sc = np.ones((3, 1, 2), dtype=np.float32)
    passed = lambda st: st not in (1, 2)      # got past host validation (no GPU here)
    assert passed(_import_status(k, k, sc))
    assert _import_status(k, k, sc, prec=2) == 1                     # AUTO is not a resolved precision
    assert _import_status(k, k, sc, mode=1) == 1                     # LOG without coefficients
    bad = k.copy(); bad[0, 1, 2, 5] = 0xFF                           # NaN code
    assert _import_status(bad, k, sc) == 1
    assert _import_status(k, bad, sc) == 1
    bad[0, 1, 2, 5] = 0x7E                                           # 448: fine
    assert passed(_import_status(bad, k, sc))
    sc2 = sc.copy(); sc2[1, 0, 1] = 0.3                              # not amax/448 of an fp16 amax
    assert _import_status(k, k, sc2) == 1
    assert "scale" in B.sdm_icl_last_error()
    sc2[1, 0, 1] = -1.0
    assert _import_status(k, k, sc2) == 1
    k16 = np.zeros((1, 2, 3, 64), dtype=np.float16)
    assert passed(_import_status(k16, k16, sc, prec=0))
    sc3 = sc.copy(); sc3[2, 0, 0] = 0.5                              # FP16 caches have unit scales
    assert _import_status(k16, k16, sc3, prec=0) == 1


def test_import_accepts_the_scale_of_every_fp16_amax():
    """fit writes s = fp32(a/448) for an fp16 amax a, for Q, K and V alike;
    import must recognise every such s (it recovers a, and with it the exact
    inverse scale)."""
    k = np.zeros((1, 1, 1, 64), dtype=np.uint8)
    a = _all_finite_fp16_positive()
    bad = []
    for i in range(a.size):
        s = icl.fp8_scale(a[i])[0]
        sc = np.full((3, 1, 1), s, dtype=np.float32)
        if _import_status(k, k, sc, lengths=(1,)) == 1:
            bad.append(float(a[i]))
    assert not bad, bad[:5]


def test_import_rejects_a_query_scale_that_is_no_amax_scale():
    """The Q slot holds s_q = fp32(amax/448) like K and V: 1.0 (an all-zero
    or 448 amax) and every fp16 amax's quotient pass; other values are
    rejected before the device."""
    k = np.zeros((1, 1, 1, 64), dtype=np.uint8)
    passed = lambda st: st not in (1, 2)
    for qs in (1.0, float(icl.fp8_scale(0.125)[0]), float(icl.fp8_scale(2.5)[0])):
        sc = np.array([[[qs]], [[0.25]], [[0.25]]], dtype=np.float32)
        assert passed(_import_status(k, k, sc, lengths=(1,)))
    for qs in (0.3, 3.01, -0.5, 0.0, np.inf, np.nan):
        sc = np.array([[[qs]], [[0.25]], [[0.25]]], dtype=np.float32)
        assert _import_status(k, k, sc, lengths=(1,)) == 1
        assert "scale" in B.sdm_icl_last_error()


def _all_finite_fp16_positive():
    v = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    return v[v > 0]


# ----------------------------------------------------------------- projection (host validation)

@pytest.mark.parametrize("kw,status", [
    (dict(in_features=48), 2),                 # not a multiple of 32
    (dict(head_dim=128), 2),
    (dict(heads=0), 1),
    (dict(scale_mode=1), 1),                   # LOG without coefficients
    (dict(scale_mode=0, gate=0x7000), 1),      # gate without GATED
    (dict(x=0x1008), 1),                       # misaligned
    (dict(q_out=None), 1),
    (dict(key_length=-1), 1),
])
def test_projection_rejects_bad_arguments(kw, status):
    a = dict(x=0x1000, w=0x2000, bias=None, batch=1, rows=10, in_features=64, heads=2, head_dim=64,
             key_length=100, head_coef=None, scale_mode=0, gate=None, q_out=0x3000, k_out=0x4000,
             v_out=0x5000, stream=None)
    a.update(kw)
    st = B.lib().sdm_icl_qkv_project(a["x"], a["w"], a["bias"], a["batch"], a["rows"], a["in_features"],
                                      a["heads"], a["head_dim"], a["key_length"], a["head_coef"],
                                      a["scale_mode"], a["gate"], a["q_out"], a["k_out"], a["v_out"], a["stream"])
    assert st == status, B.sdm_icl_last_error()
