"""Cache export -> import round trip through the C ABI: the imported cache
holds the same codes and scales and answers queries bit for bit like the
exported one (FP8 with per-batch lengths and GatedLogScale; FP16 LogScale)."""
from dataclasses import replace

import numpy as np
import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from gpu_cases import Run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("base,lengths,n_pad", [
    ("cached512k_fp8_gated", [2500, 700], 2560),
    ("ctx16k_log_fp16", [1000], 1024),
])
def test_export_import_round_trip_is_bit_exact(base, lengths, n_pad):
    import torch
    w = replace(gen.WORKLOADS[base], name="import", seed=31, n_pad=n_pad, n_valid=max(lengths),
                n_query=96, batch=len(lengths), lengths=tuple(lengths), nan_tail=True)
    r = Run(w)
    say("import round trip", base, lengths)
    cache, _ = r.fit(out_ctx=False)
    info = cache.info()
    before = r.query(cache)
    k, v, sc = B.sdm_icl_attn_cache_export(cache)
    cache.release()
    imported = B.sdm_icl_attn_cache_import(k, v, sc, lengths, w.scale_mode, info["precision"], r.coef)
    after = r.query(imported)
    torch.cuda.synchronize()
    k2, v2, sc2 = B.sdm_icl_attn_cache_export(imported)
    info2 = imported.info()
    n2, _ = B.sdm_icl_attn_cache_lengths(imported)
    imported.release()
    np.testing.assert_array_equal(before.cpu().numpy(), after.cpu().numpy())
    np.testing.assert_array_equal(k, k2)
    np.testing.assert_array_equal(v, v2)
    np.testing.assert_array_equal(sc, sc2)
    assert list(n2) == lengths
    for key in ("precision", "kv_splits", "n_valid", "keys_per_split", "length_scalar"):
        assert info[key] == info2[key], key
