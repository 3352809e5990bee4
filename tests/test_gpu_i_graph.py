"""The resident-cache query path under stream capture.

A query on a resident cache is three kernel launches into the caller's
workspace (query scaling, split-KV attention, combine): no allocation, no
copy, no synchronisation.  So it can be captured into a graph and replayed.
Each replay is compared bit for bit with the eager call on the same rows.
New query rows are copied into the captured input buffers between replays,
and eager work and synchronisations (including eager queries that reuse the
same workspace) run in between."""
from dataclasses import replace

import pytest

from long_context_tabular_amd import binding as B
from long_context_tabular_amd import inputs as gen
from gpu_cases import Run, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prec", [B.SDM_ICL_PREC_FP8_E4M3, B.SDM_ICL_PREC_FP16])
def test_query_replays_from_a_captured_graph(prec):
    import torch
    w = replace(gen.scaled_down(gen.WORKLOADS["ctx16k_gated_fp16"], 20000, 20000, 384), heads=4, seed=71,
                precision=prec, name=f"graph-{prec}")
    r = Run(w)
    say("captured query", prec)
    cache, _ = r.fit(out_ctx=False)
    try:
        R = 128
        qs = [r.qq[:, i * R:(i + 1) * R].contiguous() for i in range(3)]
        gs = [r.gq[:, i * R:(i + 1) * R].contiguous() for i in range(3)]
        ws = torch.empty(B.sdm_icl_attn_query_workspace_size(cache, R), dtype=torch.uint8, device="cuda")
        eager = []
        for q, g in zip(qs, gs):
            eager.append(B.sdm_icl_attn_query(cache, q, g, out=torch.empty_like(q), workspace=ws).clone())
        torch.cuda.synchronize()

        q_in, g_in = qs[0].clone(), gs[0].clone()
        out = torch.empty_like(q_in)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            B.sdm_icl_attn_query(cache, q_in, g_in, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            B.sdm_icl_attn_query(cache, q_in, g_in, out=out, workspace=ws)
        torch.cuda.synchronize()

        for rep in range(6):
            i = rep % 3
            q_in.copy_(qs[i])
            g_in.copy_(gs[i])
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[i]), f"replay {rep} (batch {i}) differs from the eager call"
            # eager work on the same workspace between replays
            j = (i + 1) % 3
            other = B.sdm_icl_attn_query(cache, qs[j], gs[j], out=torch.empty_like(q_in), workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[j])
        say("  6 replays bit-identical to the eager calls")
        del graph
    finally:
        cache.release()
