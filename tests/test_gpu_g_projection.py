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


def _check_unscaled_and_scaled(xd, wd, bd, gd, H, key_length, c, mode, rows=None, ref_rows=None, g=None):
    """The unscaled projection within one fp16 ulp of the oracle's (on `rows`
    or all rows), and the fused scaling bit-identical to the oracle's scaling
    of the kernel's own unscaled Q; K and V identical in both calls.  (A
    one-ulp difference of a subnormal unscaled value becomes many ulps of the
    scaled one, so the scaled output is compared on equal inputs.)"""
    import torch
    q0, k0, v0 = B.sdm_icl_qkv_project(xd, wd, bd, heads=H)
    q1, k1, v1 = B.sdm_icl_qkv_project(xd, wd, bd, heads=H, key_length=key_length,
                                       head_coef=c if mode != icl.SCALE_NONE else None, scale_mode=mode, gate=gd)
    torch.cuda.synchronize()
    sel = (lambda t: t[0, torch.from_numpy(rows).cuda()].cpu().numpy()[None]) if rows is not None else \
          (lambda t: t.cpu().numpy())
    for got, want in zip((q0, k0, v0), ref_rows):
        got = sel(got)
        diff = np.abs(got.astype(np.float32) - want.astype(np.float32))
        assert np.all(diff <= _ulp16(want) * 1.0001), float(diff.max())
        same = np.mean(got == want)
        say(f"  identical fraction {same:.5f}")
        assert same > 0.99
    np.testing.assert_array_equal(sel(k1), sel(k0))
    np.testing.assert_array_equal(sel(v1), sel(v0))
    kh = icl.head_factors(icl.length_scalar(key_length), c)
    gs = g if (g is None or rows is None) else g[:, rows]
    np.testing.assert_array_equal(sel(q1), icl.scale_queries(sel(q0), mode, kh, gs if gd is not None else None))


@pytest.mark.parametrize("R,E,H,mode", [(76833, 64, 8, icl.SCALE_LOG),      # 2 K steps: ring spans tiles
                                        (40001, 96, 3, icl.SCALE_GATED_LOG),  # 3 K steps, ragged N
                                        (30000, 32, 2, icl.SCALE_NONE)])      # 1 K step
def test_projection_many_tiles_per_workgroup(R, E, H, mode):
    """More output tiles than workgroups, so each workgroup walks several
    tiles and its load ring crosses tile boundaries; K of 1 to 3 steps of 32
    (fewer than or as many as the ring holds); ragged rows and features."""
    x, w, b, g, c = _data(1, R, E, H, 54)
    say("projection many tiles", R, E, H, mode)
    gd = to_dev(g) if mode == icl.SCALE_GATED_LOG else None
    _check_unscaled_and_scaled(to_dev(x), to_dev(w), to_dev(b), gd, H, R, c, mode,
                               ref_rows=icl.project_qkv(x, w, b, H, 64), g=g)


def test_projection_full_size_sampled_rows():
    """The benchmark's shape (524,288 hidden rows of 512 features, 8 heads,
    LogScale) in the benchmark's launch, checked on sampled rows (first and
    last rows of the range and seeded random ones) against the oracle's
    projection of those rows."""
    import torch
    M, E, H = 524288, 512, 8
    gen_t = torch.Generator(device="cuda").manual_seed(55)
    x = (torch.randn((1, M, E), generator=gen_t, device="cuda") / 2).half()
    wt = (torch.randn((3 * H * 64, E), generator=gen_t, device="cuda") / (4 * E ** 0.5)).half()
    bias = (torch.randn((3 * H * 64,), generator=gen_t, device="cuda") / 16).half()
    c = np.linspace(0.5, 1.5, H).astype(np.float32)
    rows = gen.sample_rows(M, 96, 56)
    xs = x[0, torch.from_numpy(rows).cuda()].cpu().numpy()[None]
    ref = icl.project_qkv(xs, wt.cpu().numpy(), bias.cpu().numpy(), H, 64)
    say("projection full size")
    _check_unscaled_and_scaled(x, wt, bias, None, H, M - 1000, c, icl.SCALE_LOG, rows=rows, ref_rows=ref)
