"""GPU parity of the HIP path against the float64 oracle, at sizes the oracle
finishes in seconds (several 64-key tiles, ragged tails), plus the bitwise
invariants.  All calls go through the C ABI (ctypes binding)."""
import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from oracle import icl, numerics
from tests.gpu_cases import TOL, Run, norm_err, say, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


# ----------------------------------------------------------------- K1 (bitwise)

@pytest.mark.parametrize("mode", [gen.SCALE_NONE, gen.SCALE_LOG, gen.SCALE_GATED_LOG])
def test_log_scale_bitwise(mode):
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS["ctx16k_gated_fp16"], 2000, n_query=8)
    x = gen.make_inputs(w)
    say("log_scale mode", mode)
    coef = x.head_coef if mode != gen.SCALE_NONE else None
    gate = to_dev(x.gate_ctx) if mode == gen.SCALE_GATED_LOG else None
    got = B.sdm_icl_log_scale(to_dev(x.q_ctx), 16384, coef, mode, gate=gate)
    torch.cuda.synchronize()
    kh = icl.head_factors(icl.length_scalar(16384), x.head_coef) if mode != gen.SCALE_NONE else None
    ref = icl.scale_queries(x.q_ctx[0], mode, kh, x.gate_ctx[0] if mode == gen.SCALE_GATED_LOG else None)
    np.testing.assert_array_equal(got.cpu().numpy()[0].transpose(1, 0, 2).view(np.uint16), ref.view(np.uint16))


def test_gate_exhaustive_bitwise():
    """GatedLogScale over every finite fp16 gate value (tanh pinned exhaustively)."""
    torch = _torch()
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    g = g[np.isfinite(g)]
    R, H = 7936, 8                                   # 63,488 = 7,936 x 8 gate values
    gate = g.reshape(1, R, H)
    q = np.full((1, R, H, 64), 0.3, dtype=np.float16)
    q[..., 1] = -1.7
    q[..., 2] = 6e-5                                 # an fp16 subnormal input
    coef = np.linspace(0.5, 1.5, H).astype(np.float32)
    say("gate exhaustive")
    got = B.sdm_icl_log_scale(to_dev(q), 1000, coef, gen.SCALE_GATED_LOG, gate=to_dev(gate))
    torch.cuda.synchronize()
    kh = icl.head_factors(icl.length_scalar(1000), coef)
    ref = icl.scale_queries(q[0], gen.SCALE_GATED_LOG, kh, gate[0])
    np.testing.assert_array_equal(got.cpu().numpy()[0].transpose(1, 0, 2).view(np.uint16), ref.view(np.uint16))


def test_log_scale_fp8_codes_bitwise():
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS["cached512k_fp8_gated"], 3000, n_query=8)
    x = gen.make_inputs(w)
    kh = icl.head_factors(icl.length_scalar(3000), x.head_coef)
    qt = icl.scale_queries(x.q_ctx[0], gen.SCALE_GATED_LOG, kh, x.gate_ctx[0])
    inv = np.array([icl.fp8_scale(a)[1] for a in icl.amax_rows(qt) * 0.5], dtype=np.float32)  # forces saturation
    say("log_scale fp8 codes")
    got = B.sdm_icl_log_scale(to_dev(x.q_ctx), 3000, x.head_coef, gen.SCALE_GATED_LOG,
                              gate=to_dev(x.gate_ctx), q_inv_scale=to_dev(inv.reshape(1, -1)))
    torch.cuda.synchronize()
    got = got.cpu().numpy()[0]
    for h in range(w.heads):
        np.testing.assert_array_equal(got[h], icl.quantize_codes(qt[:, h], inv[h]))


# ----------------------------------------------------------------- fit: codes and scales

@pytest.mark.parametrize("name,n_pad,n_valid", [
    ("ctx128k_fp8", 4096, 4096),
    ("model512k_fp8_log", 4096, 3096),        # NaN-filled masked tail
    ("cached512k_fp8_gated", 2050, 2050),     # ragged last tile
])
def test_fit_fp8_codes_and_scales_bitwise(name, n_pad, n_valid):
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS[name], n_pad, n_valid, n_query=8)
    r = Run(w)
    say("fit codes", name, n_pad, n_valid)
    cache, _ = r.fit(out_ctx=False)
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    info = cache.info()
    cache.release()
    o = r.oracle
    assert info["precision"] == B.SDM_ICL_PREC_FP8_E4M3 and info["n_valid"] == n_valid
    assert info["length_scalar"] == o.L32
    np.testing.assert_array_equal(sc, o.scales)
    np.testing.assert_array_equal(k, o.k_codes)
    np.testing.assert_array_equal(v, o.v_codes)


def test_fit_fp16_cache_is_a_copy():
    w = gen.scaled_down(gen.WORKLOADS["tiny_fp16"], 200, 130)
    r = Run(w)
    cache, _ = r.fit(out_ctx=False)
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    cache.release()
    np.testing.assert_array_equal(k, r.x.k_ctx[:, :130].transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(v, r.x.v_ctx[:, :130].transpose(0, 2, 1, 3))
    assert np.all(sc == 1)


# ----------------------------------------------------------------- attention parity

CASES = [
    # name, n_pad, n_valid, n_query
    ("tiny_fp16", 1024, 1024, 64),              # the tiny workload at full size
    ("tiny_fp16", 1000, 777, 33),               # ragged everything
    ("ctx16k_log_fp16", 2048, 2048, 200),
    ("ctx16k_gated_fp16", 1500, 1500, 130),
    ("ctx128k_fp8", 4096, 4096, 300),
    ("model512k_fp8_log", 3000, 2000, 256),     # NaN tail, partial tiles
    ("cached512k_fp8_gated", 2048, 2048, 129),
    ("ctx128k_fp8", 128, 100, 40),              # FP8 context of <= 128 rows (one group per wavefront)
    ("model512k_fp8_log", 320, 129, 1),         # 129 rows: one key in the last tile, one query row
    ("ctx16k_log_fp16", 128, 100, 40),          # FP16 context of <= 128 rows (one group per wavefront)
    ("ctx16k_gated_fp16", 320, 129, 3),         # FP16, two groups: one key in the last tile, one valid row
                                                # in the second wavefront's block
]


@pytest.mark.parametrize("name,n_pad,n_valid,n_query", CASES)
def test_attention_parity(name, n_pad, n_valid, n_query):
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS[name], n_pad, n_valid, n_query=n_query)
    r = Run(w)
    say("attention parity", name, n_pad, n_valid, n_query)
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    cache.release()
    out = out.cpu().numpy()[0].astype(np.float64)
    oq = oq.cpu().numpy()[0].astype(np.float64)
    tol = TOL[w.precision]
    rows = gen.sample_rows(n_valid, 600, w.seed)
    ref_c = r.ref_context(rows)
    ref_q = r.ref_query(np.arange(n_query))
    e_c, e_q = norm_err(out[rows], ref_c), norm_err(oq, ref_q)
    say(f"  context err {e_c:.3e} query err {e_q:.3e} (tol {tol})")
    assert e_c <= tol and e_q <= tol
    assert np.all(out[n_valid:] == 0)            # masked rows are zero (and not NaN)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(oq))


def test_query_rows_independent_of_batching_bitwise():
    """I6: 8 batches of 128 rows give the same bits as one batch of 1,024."""
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS["cached512k_fp8_gated"], 8192, n_query=1024)
    r = Run(w)
    say("split invariance")
    cache, _ = r.fit(out_ctx=False)
    full = r.query(cache).cpu().numpy()
    parts = np.concatenate([r.query(cache, (i, i + 128)).cpu().numpy() for i in range(0, 1024, 128)], axis=1)
    odd = np.concatenate([r.query(cache, (0, 77)).cpu().numpy(), r.query(cache, (77, 1024)).cpu().numpy()], axis=1)
    cache.release()
    np.testing.assert_array_equal(full.view(np.uint16), parts.view(np.uint16))
    np.testing.assert_array_equal(full.view(np.uint16), odd.view(np.uint16))


def test_model_call_equals_fit_then_query_and_is_deterministic():
    """I7 and I5: queries after a fit that also computed the context output
    equal queries after a cache-only fit; repeated runs are bit-identical."""
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS["model512k_fp8_log"], 4096, 3500, n_query=256)
    r = Run(w)
    say("model call vs fit+query")
    c1, out1 = r.fit(out_ctx=True)
    q1 = r.query(c1).cpu().numpy()
    c2, _ = r.fit(out_ctx=False)
    q2 = r.query(c2).cpu().numpy()
    c3, out3 = r.fit(out_ctx=True)
    q3 = r.query(c3).cpu().numpy()
    torch.cuda.synchronize()
    for c in (c1, c2, c3):
        c.release()
    np.testing.assert_array_equal(q1.view(np.uint16), q2.view(np.uint16))
    np.testing.assert_array_equal(q1.view(np.uint16), q3.view(np.uint16))
    np.testing.assert_array_equal(out1.cpu().numpy().view(np.uint16), out3.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("prec", [B.SDM_ICL_PREC_FP16, B.SDM_ICL_PREC_FP8_E4M3])
def test_closed_forms_on_gpu(prec):
    """I1 constant V gives that constant; I2 a single key gives its value row;
    I9 NaN-poisoned masked rows give the same result as zero-filled ones."""
    torch = _torch()
    rng = np.random.default_rng(9)
    N, H = 700, 2
    q = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    k = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    v = np.full((1, N, H, 64), 0.375, dtype=np.float16)
    say("closed forms", prec)
    out = torch.empty((1, N, H, 64), dtype=torch.float16, device="cuda")
    c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v), N, precision=prec, out_ctx=out)
    c.release()
    np.testing.assert_allclose(out.cpu().numpy().astype(np.float64), 0.375, rtol=0, atol=2e-4)
    # n = 1: every row returns value row 0 (exactly v0 for FP16; code * s_v for FP8)
    v1 = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v1), 1, precision=prec, out_ctx=out)
    got = out.cpu().numpy()[0, 0].astype(np.float64)
    ref = icl.fit(q, k, v1, 1, icl.SCALE_NONE, prec)
    want = np.stack([ref.vhat(0, h)[0] for h in range(H)])
    c.release()
    np.testing.assert_allclose(got, want, rtol=1e-3, atol=1e-7)
    # NaN tail vs zero tail
    qn, kn, vn = q.copy(), k.copy(), v1.copy()
    for t in (qn, kn, vn):
        t[:, 500:] = np.float16(np.nan)
    qz, kz, vz = q.copy(), k.copy(), v1.copy()
    for t in (qz, kz, vz):
        t[:, 500:] = 0
    o_n = torch.empty_like(out)
    o_z = torch.empty_like(out)
    c1 = B.sdm_icl_attn_fit(to_dev(qn), to_dev(kn), to_dev(vn), 500, precision=prec, out_ctx=o_n)
    c2 = B.sdm_icl_attn_fit(to_dev(qz), to_dev(kz), to_dev(vz), 500, precision=prec, out_ctx=o_z)
    c1.release()
    c2.release()
    np.testing.assert_array_equal(o_n.cpu().numpy().view(np.uint16), o_z.cpu().numpy().view(np.uint16))


def test_query_misuse_and_workspace_errors():
    import ctypes
    torch = _torch()
    w = gen.scaled_down(gen.WORKLOADS["ctx16k_gated_fp16"], 256, n_query=16)
    r = Run(w)
    cache, _ = r.fit(out_ctx=False)
    with pytest.raises(B.SdmIclError) as e:
        B.sdm_icl_attn_query(cache, r.qq)                  # gated cache, no gate
    assert e.value.status == 1
    need = B.sdm_icl_attn_query_workspace_size(cache, 16)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SdmIclError) as e:
        B.sdm_icl_attn_query(cache, r.qq, r.gq, workspace=small)
    assert e.value.status == 6
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(r.qq)
    host_q = np.ascontiguousarray(r.x.q_query)
    st = B.lib().sdm_icl_attn_query(cache.handle, host_q.ctypes.data, r.gq.data_ptr(), 16,
                                    out.data_ptr(), ws.data_ptr(), need, None)
    assert st == 3, B.sdm_icl_last_error()             # host memory is rejected before launch
    h = cache.handle
    cache.release()
    assert B.lib().sdm_icl_attn_release(ctypes.c_void_p(h)) == 6   # double release
    assert B.lib().sdm_icl_attn_query(ctypes.c_void_p(h), r.qq.data_ptr(), r.gq.data_ptr(), 16,
                                      out.data_ptr(), ws.data_ptr(), need, None) == 6


def test_auto_precision_follows_threshold():
    for n, want in ((8192, B.SDM_ICL_PREC_FP16), (8193, B.SDM_ICL_PREC_FP8_E4M3)):
        w = gen.scaled_down(gen.WORKLOADS["tiny_fp16"], n, n, n_query=4)
        r = Run(w)
        c = B.sdm_icl_attn_fit(r.q, r.k, r.v, n, precision=B.SDM_ICL_PREC_AUTO)
        assert c.info()["precision"] == want
        c.release()


@pytest.mark.parametrize("prec", [B.SDM_ICL_PREC_FP16, B.SDM_ICL_PREC_FP8_E4M3])
def test_reference_moves_when_later_tiles_dominate(prec):
    """Keys whose scale grows along the context make later tiles' scores
    exceed a row's first-tile reference by far, so the reference-moving path
    runs many times; near-zero queries (every other row) never trigger it.
    Parity with the oracle, and bitwise batch-split invariance for rows whose
    neighbours take that path."""
    torch = _torch()
    rng = np.random.default_rng(21)
    N, H, R = 2048, 2, 64
    growth = (1.0 + np.arange(N) / 35.0)[None, :, None, None]
    q = (rng.standard_normal((1, N, H, 64))).astype(np.float16)
    k = (rng.standard_normal((1, N, H, 64)) * growth / 8).astype(np.float16)
    v = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    qq = (rng.standard_normal((1, R, H, 64))).astype(np.float16)
    q[:, 1::2] *= np.float16(1e-3)
    qq[:, 1::2] *= np.float16(1e-3)
    say("reference moves", prec)
    out = torch.empty((1, N, H, 64), dtype=torch.float16, device="cuda")
    c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v), N, precision=prec, out_ctx=out)
    full = B.sdm_icl_attn_query(c, to_dev(qq)).cpu().numpy()
    halves_ = np.concatenate([B.sdm_icl_attn_query(c, to_dev(qq[:, :32])).cpu().numpy(),
                              B.sdm_icl_attn_query(c, to_dev(qq[:, 32:])).cpu().numpy()], axis=1)
    torch.cuda.synchronize()
    c.release()
    np.testing.assert_array_equal(full.view(np.uint16), halves_.view(np.uint16))
    ref = icl.fit(q, k, v, N, icl.SCALE_NONE, prec)
    rows = np.concatenate([np.arange(0, 64), np.arange(N - 64, N)])
    e_c = norm_err(out.cpu().numpy()[0, rows].astype(np.float64), icl.context_outputs(ref, q, None, rows))
    e_q = norm_err(full[0].astype(np.float64), icl.attend(ref, qq[0], None))
    say(f"  context err {e_c:.3e} query err {e_q:.3e}")
    assert e_c <= TOL[prec] and e_q <= TOL[prec]


@pytest.mark.parametrize("prec", [B.SDM_ICL_PREC_FP16, B.SDM_ICL_PREC_FP8_E4M3])
def test_rows_beside_a_moving_reference_keep_their_bits(prec):
    """Only query rows 0..9 meet a key far above their first-tile reference
    (they point at key 1,500), so they move it; rows 10.. have logits with a
    spread of a few log2 units that never overflow.  Split at rows 10 and 20
    (not multiples of the 32-row groups), rows 10..31 share a group with the
    moving rows in one launch and not in the other: their bits must not
    change."""
    torch = _torch()
    rng = np.random.default_rng(23)
    N, H, R = 2048, 2, 96
    k = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    v = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    qq = (rng.standard_normal((1, R, H, 64)) * 16).astype(np.float16)
    target = k[0, 1500].astype(np.float64)
    qq[0, :10] = (200.0 * target / np.linalg.norm(target, axis=-1, keepdims=True)).astype(np.float16)
    q = (rng.standard_normal((1, N, H, 64)) * 16).astype(np.float16)
    q[0, 0, :, 0] = 250                              # context Q amax above every query element
    say("rows beside a moving reference", prec)
    c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v), N, precision=prec)
    full = B.sdm_icl_attn_query(c, to_dev(qq)).cpu().numpy()
    for cut in (10, 20):
        parts = np.concatenate([B.sdm_icl_attn_query(c, to_dev(qq[:, :cut])).cpu().numpy(),
                                B.sdm_icl_attn_query(c, to_dev(qq[:, cut:])).cpu().numpy()], axis=1)
        np.testing.assert_array_equal(full.view(np.uint16), parts.view(np.uint16))
    torch.cuda.synchronize()
    c.release()
    ref = icl.fit(q, k, v, N, icl.SCALE_NONE, prec)
    e_q = norm_err(full[0].astype(np.float64), icl.attend(ref, qq[0], None))
    say(f"  query err {e_q:.3e}")
    assert e_q <= TOL[prec]


def test_fp8_query_rows_above_the_context_amax_saturate():
    """Query rows reuse the context's Q scale: elements beyond the context
    amax saturate at it (the method's +-448 codes).  Queries drawn 32x wider
    than the context's Q saturate in most elements; the result follows the
    oracle's saturated rows."""
    torch = _torch()
    rng = np.random.default_rng(29)
    N, H, R = 1500, 2, 100
    q = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    k = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    v = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    qq = (rng.standard_normal((1, R, H, 64)) * 4).astype(np.float16)
    say("fp8 query saturation")
    c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v), N, precision=B.SDM_ICL_PREC_FP8_E4M3)
    got = B.sdm_icl_attn_query(c, to_dev(qq)).cpu().numpy()[0].astype(np.float64)
    torch.cuda.synchronize()
    c.release()
    ref = icl.fit(q, k, v, N, icl.SCALE_NONE, icl.PREC_FP8_E4M3)
    frac = np.mean(np.abs(qq[0].astype(np.float64)) > icl.amax_rows(q[0])[None, :, None])
    want = icl.attend(ref, qq[0], None)
    err = norm_err(got, want)
    say(f"  saturated fraction {frac:.2f}, normalised error {err:.2e}")
    assert frac > 0.5
    assert err <= TOL[B.SDM_ICL_PREC_FP8_E4M3]


def test_fp8_query_scale_edges():
    """The FP8 Q scale at its edges: an all-zero Q (unit scales; every key
    equally weighted, so each row returns the mean of the dequantised V) and
    large-magnitude queries against tiny keys (a logit factor s_q s_k / 8 far
    from 1), each against the oracle."""
    torch = _torch()
    rng = np.random.default_rng(71)
    N, H = 300, 2
    k = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    v = (rng.standard_normal((1, N, H, 64)) / 8).astype(np.float16)
    cases = {
        "zero q": (np.zeros((1, N, H, 64), dtype=np.float16), k),
        "large q, tiny k": ((rng.standard_normal((1, N, H, 64)) * 8000).clip(-65000, 65000).astype(np.float16),
                            (k.astype(np.float32) * 1e-3).astype(np.float16)),
    }
    for name, (q, kk) in cases.items():
        say("q scale edge:", name)
        out = torch.empty((1, N, H, 64), dtype=torch.float16, device="cuda")
        c = B.sdm_icl_attn_fit(to_dev(q), to_dev(kk), to_dev(v), N, precision=B.SDM_ICL_PREC_FP8_E4M3, out_ctx=out)
        _, _, sc = B.sdm_icl_attn_cache_export(c)
        c.release()
        ref = icl.fit(q, kk, v, N, icl.SCALE_NONE, icl.PREC_FP8_E4M3)
        np.testing.assert_array_equal(sc, ref.scales)
        rows = np.arange(N)
        want = icl.context_outputs(ref, q, None, rows)
        got = out.cpu().numpy()[0].astype(np.float64)
        err = norm_err(got, want)
        say(f"  normalised error {err:.2e}, s_q {sc[0, 0, 0]!r}")
        assert err <= TOL[B.SDM_ICL_PREC_FP8_E4M3]
        if name == "zero q":
            assert sc[0, 0, 0] == 1.0
            mean_v = np.stack([ref.vhat(0, h).mean(axis=0) for h in range(H)])
            np.testing.assert_allclose(got, np.broadcast_to(mean_v, got.shape), rtol=0, atol=2e-3 * np.abs(mean_v).max())


def test_fp8_path_equals_fp16_path_on_grid_inputs():
    """I10 on the GPU: Q~, K and V drawn from the e4m3 grid times a
    power-of-two scale per tensor and head (amax pinned to 448 s), so FP8
    quantisation is lossless: the oracle's FP8 and FP16 results are
    identical, and the kernels' K/V codes and the exported scales must be
    exactly the grid's.  The GPU's FP8 path then differs from its FP16 path
    only in fp32 rounding of the scores (sums of code products times
    s_q s_k against sums of fp16 products), so the two must agree within the
    FP16 tolerance, far inside the FP8 one.  One head has tiny logits, the
    other a spread of about 0.8."""
    torch = _torch()
    rng = np.random.default_rng(31)
    N, H, R = 640, 2, 96
    grid = numerics.E4M3_VALUES[np.isfinite(numerics.E4M3_VALUES)]
    grid = grid[np.abs(grid) <= 64]
    scales = {"q": (2.0 ** -9, 2.0 ** -3), "k": (2.0 ** -10, 2.0 ** -5), "v": (2.0 ** -6, 2.0 ** -11)}
    amax_dim = {"q": 0, "k": 1, "v": 2}     # the pinned amax elements never meet in a dot product

    def draw(name, rows):
        t = np.empty((1, rows, H, 64))
        for h in range(H):
            t[0, :, h] = rng.choice(grid, size=(rows, 64)) * scales[name][h]
            t[0, 0, h, amax_dim[name]] = 448 * scales[name][h]
        assert np.all(t.astype(np.float16).astype(np.float64) == t)
        return t.astype(np.float16)

    q, k, v = draw("q", N), draw("k", N), draw("v", N)
    qq = draw("q", R)
    qq[0, 0] = qq[0, 1]                     # query rows stay within the context amax
    say("I10 grid inputs")
    outs = {}
    for prec in (B.SDM_ICL_PREC_FP16, B.SDM_ICL_PREC_FP8_E4M3):
        out = torch.empty((1, N, H, 64), dtype=torch.float16, device="cuda")
        c = B.sdm_icl_attn_fit(to_dev(q), to_dev(k), to_dev(v), N, precision=prec, out_ctx=out)
        oq = B.sdm_icl_attn_query(c, to_dev(qq))
        if prec == B.SDM_ICL_PREC_FP8_E4M3:
            kc, vc, sc = B.sdm_icl_attn_cache_export(c)
        torch.cuda.synchronize()
        c.release()
        outs[prec] = (out.cpu().numpy()[0].astype(np.float64), oq.cpu().numpy()[0].astype(np.float64))
    ref8 = icl.fit(q, k, v, N, icl.SCALE_NONE, icl.PREC_FP8_E4M3)
    ref16 = icl.fit(q, k, v, N, icl.SCALE_NONE, icl.PREC_FP16)
    for t, name in enumerate("qkv"):
        np.testing.assert_array_equal(sc[t, 0], np.float32(scales[name]))
    np.testing.assert_array_equal(kc, ref8.k_codes)
    np.testing.assert_array_equal(vc, ref8.v_codes)
    for which, rows_q in ((0, q[0]), (1, qq[0])):
        want = icl.attend(ref16, rows_q, None)
        assert np.array_equal(icl.attend(ref8, rows_q, None), want)
        o16, o8 = outs[B.SDM_ICL_PREC_FP16][which], outs[B.SDM_ICL_PREC_FP8_E4M3][which]
        for h in range(H):
            e_paths = norm_err(o8[:, h], o16[:, h])
            e8, e16 = norm_err(o8[:, h], want[:, h]), norm_err(o16[:, h], want[:, h])
            say(f"  {'context' if which == 0 else 'query'} head {h}: FP8 vs FP16 path {e_paths:.2e}, "
                f"FP8 vs oracle {e8:.2e}, FP16 vs oracle {e16:.2e}")
            assert e_paths <= TOL[B.SDM_ICL_PREC_FP16]
            assert e8 <= TOL[B.SDM_ICL_PREC_FP16] and e16 <= TOL[B.SDM_ICL_PREC_FP16]
