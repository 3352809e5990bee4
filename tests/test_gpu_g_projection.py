"""The Q/K/V projection with the query scaling fused into its epilogue,
through the C ABI: parity with the float64 oracle (one fp16 rounding of the
exact sum; the kernel accumulates in float32, so it may differ by one fp16
unit in the last place), the fused scaling bit-identical to the separate
scaling pass on the kernel's own unscaled projection, and the projected
rows feeding fit and query."""
import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from oracle import icl
from gpu_cases import TOL, norm_err, say, to_dev

pytestmark = pytest.mark.gpu


def _data(Bn, R, E, H, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((Bn, R, E)) / 2).astype(np.float16)
    w = (rng.standard_normal((3 * H * 64, E)) / np.sqrt(E) / 4).astype(np.float16)
    b = (rng.standard_normal(3 * H * 64) / 16).astype(np.float16)
    g = rng.standard_normal((Bn, R, H)).astype(np.float16)
    c = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    return x, w, b, g, c


def _ulp16(a):
    a = np.abs(a.astype(np.float32))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("Bn,R,E,H", [(2, 300, 512, 8), (1, 77, 96, 3)])
def test_projection_matches_oracle_within_one_ulp(Bn, R, E, H):
    import torch
    x, w, b, g, c = _data(Bn, R, E, H, 51)
    say("projection parity", Bn, R, E, H)
    q, k, v = B.sdm_icl_qkv_project(to_dev(x), to_dev(w), to_dev(b), heads=H)
    torch.cuda.synchronize()
    ref = icl.project_qkv(x, w, b, H, 64)
    for got, want in zip((q, k, v), ref):
        got = got.cpu().numpy()
        diff = np.abs(got.astype(np.float32) - want.astype(np.float32))
        assert np.all(diff <= _ulp16(want) * 1.0001), float(diff.max())
        same = np.mean(got == want)
        say(f"  identical fraction {same:.5f}")
        assert same > 0.99


@pytest.mark.parametrize("mode", [icl.SCALE_LOG, icl.SCALE_GATED_LOG])
def test_fused_scaling_equals_the_separate_pass_bitwise(mode):
    import torch
    Bn, R, E, H = 2, 260, 512, 8
    x, w, b, g, c = _data(Bn, R, E, H, 52)
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    gd = to_dev(g) if mode == icl.SCALE_GATED_LOG else None
    q0, k0, v0 = B.sdm_icl_qkv_project(xd, wd, bd, heads=H)
    q1, k1, v1 = B.sdm_icl_qkv_project(xd, wd, bd, heads=H, key_length=40000, head_coef=c,
                                       scale_mode=mode, gate=gd)
    sep = B.sdm_icl_log_scale(q0, 40000, c, mode, gate=gd)          # head-major [B, H, R, D]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q1.cpu().numpy(), sep.cpu().numpy().transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(k1.cpu().numpy(), k0.cpu().numpy())
    np.testing.assert_array_equal(v1.cpu().numpy(), v0.cpu().numpy())
    kh = icl.head_factors(icl.length_scalar(40000), c)
    np.testing.assert_array_equal(
        q1.cpu().numpy(), icl.scale_queries(q0.cpu().numpy(), mode, kh, g if gd is not None else None))


def test_projected_rows_feed_fit_and_query():
    """Hidden rows -> fused projection (GatedLogScale) -> fit(NONE, FP8) with
    the context self-attention -> query; against the oracle run on the
    oracle's own projection of the same rows."""
    import torch
    n, R, E, H = 3000, 96, 512, 8
    x, w, b, g, c = _data(1, n + R, E, H, 53)
    xd, wd, bd, gd = to_dev(x), to_dev(w), to_dev(b), to_dev(g)
    q, k, v = B.sdm_icl_qkv_project(xd, wd, bd, heads=H, key_length=n, head_coef=c,
                                    scale_mode=icl.SCALE_GATED_LOG, gate=gd)
    qc, kc, vc = q[:, :n].contiguous(), k[:, :n].contiguous(), v[:, :n].contiguous()
    out = torch.empty_like(qc)
    cache = B.sdm_icl_attn_fit(qc, kc, vc, n, B.SDM_ICL_SCALE_NONE, B.SDM_ICL_PREC_FP8_E4M3, out_ctx=out)
    oq = B.sdm_icl_attn_query(cache, q[:, n:].contiguous())
    torch.cuda.synchronize()
    cache.release()
    kh = icl.head_factors(icl.length_scalar(n), c)
    rq, rk, rv = icl.project_scaled(x, w, b, H, 64, icl.SCALE_GATED_LOG, kh, g)
    o = icl.fit(rq[:, :n], rk[:, :n], rv[:, :n], n, icl.SCALE_NONE, icl.PREC_FP8_E4M3)
    rows = gen.sample_rows(n, 64, 9)
    e_ctx = norm_err(out.cpu().numpy()[0, rows], icl.context_outputs(o, rq[:, :n], None, rows))
    e_q = norm_err(oq.cpu().numpy()[0], icl.attend(o, rq[0, n:], None))
    say(f"projected rows: context err {e_ctx:.2e}, query err {e_q:.2e}")
    assert e_ctx <= TOL[B.SDM_ICL_PREC_FP8_E4M3] and e_q <= TOL[B.SDM_ICL_PREC_FP8_E4M3]
