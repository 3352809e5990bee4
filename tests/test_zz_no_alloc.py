"""The no-allocation query entry point (sdm_icl_attn_query_noalloc) against
the workspace entry point (sdm_icl_attn_query) through the C ABI: the same
bits on two calls in a row on one GPU's scratch array, the second with fewer
rows, both also within tolerance of the float64 oracle; sizes beyond the
scratch array and offloaded caches are rejected before anything is
launched."""
import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from tests.gpu_cases import TOL, Run, norm_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,n_pad,rows", [
    ("cached512k_fp8_gated", 16384, (200, 77)),      # FP8, GatedLogScale, 64 KV splits
    ("ctx16k_log_fp16", 6000, (129, 1)),             # FP16, LogScale, ragged last key tile
])
def test_noalloc_query_equals_the_workspace_query(name, n_pad, rows):
    import torch
    w = gen.scaled_down(gen.WORKLOADS[name], n_pad, n_query=max(rows))
    r = Run(w)
    say("noalloc", name, n_pad, rows)
    cache, _ = r.fit(out_ctx=False)
    for R in rows:                                   # the second call has fewer rows
        q = r.qq[:, :R].contiguous()
        g = r.gq[:, :R].contiguous() if r.gq is not None else None
        want = B.sdm_icl_attn_query(cache, q, g)
        got = torch.full_like(q, float("nan"))
        B.sdm_icl_attn_query_noalloc(cache, q, g, out=got)
        torch.cuda.synchronize()
        want, got = want.cpu().numpy(), got.cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))
        err = norm_err(got[0].astype(np.float64), r.ref_query(np.arange(R)))
        say(f"  R={R}: bit-identical to the workspace query; normalised error {err:.2e}")
        assert err <= TOL[w.precision]
    cache.release()


def test_noalloc_query_rejects_what_the_scratch_cannot_hold():
    import torch
    w = gen.scaled_down(gen.WORKLOADS["cached512k_fp8_gated"], 16384, n_query=1024)
    r = Run(w)
    say("noalloc limits")
    cache, _ = r.fit(out_ctx=False)
    need = B.sdm_icl_attn_query_workspace_size(cache, 1024)
    assert need > B.SDM_ICL_NOALLOC_SCRATCH_BYTES
    out = torch.full_like(r.qq, 7.0)
    with pytest.raises(B.SdmIclError) as e:
        B.sdm_icl_attn_query_noalloc(cache, r.qq, r.gq, out=out)
    assert e.value.status == 1 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))               # nothing was launched
    B.sdm_icl_attn_cache_offload(cache)
    q = r.qq[:, :16].contiguous()
    g = r.gq[:, :16].contiguous()
    with pytest.raises(B.SdmIclError) as e:
        B.sdm_icl_attn_query_noalloc(cache, q, g)
    assert e.value.status == 2 and "offloaded" in str(e.value)
    cache.release()
