"""The split-KV combine across its chunk boundaries, through the C ABI.

The split plan gives about 3 (split, head) units per CU over all (b, h) with at least
4 key tiles per split, so with 2 heads and one batch element n = 16,384 /
16,640 / 32,768 / 33,000 / 70,000 rows give 64 / 65 / 128 / 129 / 274 splits
on a 256-CU MI355X.  The combine takes up to 128 splits in one pass and more
in chunks of 64; the cases cover one chunk, a ragged second chunk, exactly
two chunks, the first row count past the single pass, and many chunks.
Parity per element with the float64 oracle on every query row (FP16, the
tighter bound), and a query batch split two ways stays bit-identical."""
from dataclasses import replace

import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from gpu_cases import TOL, Run, norm_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,expect_splits", [(16384, 64), (16640, 65), (32768, 128), (33000, 129), (70000, 274)])
def test_combine_chunk_boundaries(n, expect_splits):
    import torch
    w = replace(gen.scaled_down(gen.WORKLOADS["ctx16k_gated_fp16"], n, n, 37), heads=2, seed=61,
                name=f"splits{n}")
    r = Run(w)
    say("combine boundaries", n, expect_splits)
    cache, _ = r.fit(out_ctx=False)
    try:
        info = B.sdm_icl_attn_cache_info(cache)
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert info["kv_splits"] == expect_splits
        assert info["precision"] == B.SDM_ICL_PREC_FP16
        whole = r.query(cache).cpu().numpy()
        parts = np.concatenate([r.query(cache, (0, 13)).cpu().numpy(), r.query(cache, (13, 37)).cpu().numpy()],
                               axis=1)
        torch.cuda.synchronize()
    finally:
        cache.release()
    np.testing.assert_array_equal(whole, parts)
    err = norm_err(whole[0], r.ref_query(np.arange(37)))
    say(f"  splits {info['kv_splits']}: normalised error {err:.2e}")
    assert err <= TOL[B.SDM_ICL_PREC_FP16]


@pytest.mark.parametrize("base,prec", [("ctx16k_gated_fp16", B.SDM_ICL_PREC_FP8_E4M3),
                                       ("ctx16k_log_fp16", B.SDM_ICL_PREC_FP16)])
def test_xcd_order_with_a_partial_group_of_units(base, prec):
    """Several query-row blocks per KV split run back to back on one XCD; with
    3 heads the (split, head) units are not a multiple of 8, so the last ones
    take the plain order.  300 query rows are 2 row blocks (FP8, 256 rows) or 3
    (FP16, 128 rows) in one launch; the same rows queried as 137 + 163 are one
    block per launch.  Both must agree bit for bit, and with the oracle."""
    import torch
    w = replace(gen.scaled_down(gen.WORKLOADS[base], 20000, 20000, 300), heads=3, seed=67, precision=prec,
                name=f"xcd-tail-{prec}")
    r = Run(w)
    say("xcd order, partial group of units", base, prec)
    cache, _ = r.fit(out_ctx=False)
    try:
        info = B.sdm_icl_attn_cache_info(cache)
        units = info["kv_splits"] * 3
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert units % 8 != 0
        whole = r.query(cache).cpu().numpy()
        parts = np.concatenate([r.query(cache, (0, 137)).cpu().numpy(), r.query(cache, (137, 300)).cpu().numpy()],
                               axis=1)
        torch.cuda.synchronize()
    finally:
        cache.release()
    np.testing.assert_array_equal(whole, parts)
    err = norm_err(whole[0], r.ref_query(np.arange(300)))
    say(f"  splits {info['kv_splits']} ({units} units): normalised error {err:.2e}")
    assert err <= TOL[prec]
