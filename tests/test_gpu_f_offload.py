"""Host offload and chunked streaming through the C ABI ("[FP8 3/4] Integrate
FP8 attention and caching into TabICLv2", introduction: cache chunking and
CPU offloading are supported): queries on an offloaded cache stream K/V from
pinned host memory chunk by chunk and give, bit for bit, what the resident
cache gives."""
from dataclasses import replace

import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from gpu_cases import Run, TOL, norm_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("base,lengths,n_pad,chunk", [
    ("cached512k_fp8_gated", [24000, 3000], 24576, 1_000_000), # several chunks, ragged last chunk, empty splits
    ("cached512k_fp8_gated", [5000], 5120, 0),                 # default chunk: one chunk
    ("ctx16k_log_fp16", [9000], 9216, 600_000),                # FP16 cache
])
def test_offloaded_queries_are_bit_identical(base, lengths, n_pad, chunk):
    import torch
    w = replace(gen.WORKLOADS[base], name="offload", seed=41, n_pad=n_pad, n_valid=max(lengths),
                n_query=160, batch=len(lengths), lengths=tuple(lengths), nan_tail=True)
    r = Run(w)
    say("offload", base, lengths, chunk)
    cache, _ = r.fit(out_ctx=False)
    resident = [r.query(cache), r.query(cache, (0, 37))]
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    full_bytes = cache.info()["device_bytes"]
    B.sdm_icl_attn_cache_offload(cache, chunk)
    info = cache.info()
    say("  offloaded:", info["offloaded"], "chunk splits", info["stream_chunk_splits"], "of", info["kv_splits"],
        "device bytes", info["device_bytes"], "of", full_bytes)
    assert info["offloaded"] == 1 and info["device_bytes"] < full_bytes // 100
    if chunk:
        assert info["stream_chunk_splits"] < info["kv_splits"]        # more than one chunk
    streamed = [r.query(cache), r.query(cache, (0, 37))]
    k2, v2, sc2 = B.sdm_icl_attn_cache_export(cache)
    B.sdm_icl_attn_cache_restore(cache)
    assert cache.info()["offloaded"] == 0 and cache.info()["device_bytes"] == full_bytes
    back = [r.query(cache), r.query(cache, (0, 37))]
    torch.cuda.synchronize()
    for a, b2, c in zip(resident, streamed, back):
        np.testing.assert_array_equal(a.cpu().numpy(), b2.cpu().numpy())
        np.testing.assert_array_equal(a.cpu().numpy(), c.cpu().numpy())
    np.testing.assert_array_equal(k, k2)
    np.testing.assert_array_equal(v, v2)
    np.testing.assert_array_equal(sc, sc2)
    # and the streamed result is the oracle's
    got = streamed[0].cpu().numpy()
    for b, nb in enumerate(lengths):
        rows = np.arange(0, 160, 9)
        e = norm_err(got[b, rows], r.ref_query(rows, b=b))
        say(f"  b={b}: err {e:.2e}")
        assert e <= TOL[w.precision]
    B.sdm_icl_attn_cache_offload(cache, chunk)      # releasing an offloaded cache frees host memory too
    cache.release()
