"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses.  Outputs are compared element by element with the float64
oracle (each row against all n keys): every row of the tiny and the 16K
workloads, every query row of the others, and seeded samples of context rows
(2,048 at 128K; 1,024 valid rows, including the first and last 8, at 512K
and per element of the ragged 128K + 64K pair);
FP8 codes and scales bitwise; and the bitwise invariants at full size.  The
oracle runs on the host's cores, one head and a share of the rows per
thread."""
import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from tests.gpu_cases import TOL, Run, norm_err, say

pytestmark = pytest.mark.gpu


def _check(run, out_ctx, out_q, ctx_rows, q_rows):
    w = run.w
    tol = TOL[w.precision]
    e_c = e_q = 0.0
    if out_ctx is not None and len(ctx_rows):
        ref = run.ref_context(ctx_rows)
        e_c = norm_err(out_ctx[0, ctx_rows].astype(np.float64), ref)
    if out_q is not None and len(q_rows):
        ref = run.ref_query(q_rows)
        e_q = norm_err(out_q[0, q_rows].astype(np.float64), ref)
    say(f"  {w.name}: context err {e_c:.3e}, query err {e_q:.3e} (tol {tol})")
    assert e_c <= tol and e_q <= tol


@pytest.mark.timeout(600)
def test_full_tiny_fp16():
    import torch
    r = Run(gen.WORKLOADS["tiny_fp16"])
    say("full tiny_fp16")
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    cache.release()
    _check(r, out.cpu().numpy(), oq.cpu().numpy(), np.arange(1024), np.arange(64))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["ctx16k_log_fp16", "ctx16k_gated_fp16"])
def test_full_ctx16k(name):
    import torch
    r = Run(gen.WORKLOADS[name])
    say("full", name)
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    cache.release()
    _check(r, out.cpu().numpy(), oq.cpu().numpy(), np.arange(16384), np.arange(1024))


@pytest.mark.timeout(600)
def test_full_ctx128k_fp8():
    import torch
    r = Run(gen.WORKLOADS["ctx128k_fp8"])
    say("full ctx128k_fp8")
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    cache.release()
    o = r.oracle
    np.testing.assert_array_equal(sc, o.scales)
    np.testing.assert_array_equal(k, o.k_codes)
    np.testing.assert_array_equal(v, o.v_codes)
    _check(r, out.cpu().numpy(), oq.cpu().numpy(), gen.sample_rows(131072, 2048, 2), np.arange(1024))


@pytest.mark.timeout(600)
def test_full_cached512k_fp8_gated():
    """Cached prediction against a resident 524,288-row FP8 cache: sampled
    parity, and 8 x 128 query batches bit-identical to 1 x 1,024."""
    import torch
    r = Run(gen.WORKLOADS["cached512k_fp8_gated"], oracle_codes=True)
    say("full cached512k_fp8_gated")
    cache, _ = r.fit(out_ctx=False)
    full = r.query(cache).cpu().numpy()
    parts = np.concatenate([r.query(cache, (i, i + 128)).cpu().numpy() for i in range(0, 1024, 128)], axis=1)
    torch.cuda.synchronize()
    _, _, sc = B.sdm_icl_attn_cache_export(cache)
    # the same queries with the cache offloaded to host memory and streamed
    # back in chunks (default chunk size): bit-identical
    B.sdm_icl_attn_cache_offload(cache)
    info = cache.info()
    say(f"  offloaded: {info['stream_chunk_splits']} of {info['kv_splits']} splits per chunk")
    streamed = r.query(cache).cpu().numpy()
    streamed128 = r.query(cache, (384, 512)).cpu().numpy()
    cache.release()
    assert info["offloaded"] == 1 and info["stream_chunk_splits"] < info["kv_splits"]
    np.testing.assert_array_equal(full.view(np.uint16), parts.view(np.uint16))
    np.testing.assert_array_equal(full.view(np.uint16), streamed.view(np.uint16))
    np.testing.assert_array_equal(full[:, 384:512].view(np.uint16), streamed128.view(np.uint16))
    np.testing.assert_array_equal(sc, r.oracle.scales)
    _check(r, None, full, [], np.arange(1024))


@pytest.mark.timeout(600)
def test_full_model512k_fp8_log():
    """Full model call at 524,288 padded rows (last 1,000 masked, NaN-filled)."""
    import torch
    w = gen.WORKLOADS["model512k_fp8_log"]
    r = Run(w)
    say("full model512k_fp8_log")
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    info = cache.info()
    cache.release()
    out = out.cpu().numpy()
    assert info["n_valid"] == 523288 and info["length_scalar"] == r.oracle.L32
    assert np.all(out[0, w.n_valid:] == 0)
    _check(r, out, oq.cpu().numpy(), gen.sample_rows(w.n_valid, 1024, w.seed), np.arange(1024))


@pytest.mark.timeout(600)
def test_full_ragged128k_fp8():
    """The ragged pair the benchmark times (131,072 and 65,537 valid rows of
    131,072 in one fit and one query launch, FP8, outliers, NaN past each
    length): codes and scales bitwise, 1,024 sampled context rows of each
    element (its first and last 8 included) and all 1,024 queries of each,
    against all of that element's keys; the masked rows of the short element
    exactly zero."""
    import torch
    w = gen.WORKLOADS["ragged128k_fp8"]
    r = Run(w)
    say("full ragged128k_fp8")
    cache, out = r.fit(out_ctx=True)
    oq = r.query(cache)
    torch.cuda.synchronize()
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    n_b, _ = B.sdm_icl_attn_cache_lengths(cache)
    cache.release()
    assert list(n_b) == [131072, 65537]
    o = r.oracle
    np.testing.assert_array_equal(sc, o.scales)
    for b, n in enumerate((131072, 65537)):
        np.testing.assert_array_equal(k[b, :, :n], o.k_codes_b[b])
        np.testing.assert_array_equal(v[b, :, :n], o.v_codes_b[b])
        assert not np.any(k[b, :, n:]) and not np.any(v[b, :, n:])
    out, oq = out.cpu().numpy(), oq.cpu().numpy()
    assert not np.any(out[1, 65537:])
    tol = TOL[w.precision]
    for b, n in enumerate((131072, 65537)):
        rows = gen.sample_rows(n, 1024, 70 + b)
        e_c = norm_err(out[b, rows].astype(np.float64), r.ref_context(rows, b=b))
        e_q = norm_err(oq[b].astype(np.float64), r.ref_query(np.arange(1024), b=b))
        say(f"  b={b} (n={n}): context err {e_c:.3e}, query err {e_q:.3e} (tol {tol})")
        assert e_c <= tol and e_q <= tol


@pytest.mark.timeout(600)
def test_full_ragged_two_contexts_in_one_cache():
    """Two batch elements with 524,288 and 300,001 valid rows in one fit and
    one query launch (per-batch lengths, FP8, GatedLogScale, outliers, NaN
    tails): sampled parity per element, each against all of its keys."""
    import torch
    from dataclasses import replace
    w = replace(gen.WORKLOADS["cached512k_fp8_gated"], name="ragged512k", seed=61, batch=2,
                lengths=(524288, 300001), n_query=256, nan_tail=True)
    r = Run(w)
    say("full ragged 524,288 + 300,001")
    cache, _ = r.fit(out_ctx=False)
    oq = r.query(cache).cpu().numpy()
    n_b, L = B.sdm_icl_attn_cache_lengths(cache)
    cache.release()
    assert list(n_b) == [524288, 300001]
    np.testing.assert_array_equal(L, r.oracle.L32s)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(252, 256), np.arange(5, 256, 41)]))
    for b in range(2):
        e = norm_err(oq[b, rows].astype(np.float64), r.ref_query(rows, b=b))
        say(f"  b={b}: query err {e:.3e}")
        assert e <= TOL[w.precision]
