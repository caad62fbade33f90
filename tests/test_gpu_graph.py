"""Decode and prefill captured in a HIP graph give the eager results on every replay."""
import pytest
import torch

import gqa_attention_amd as g
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads.generate import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_available):
    dinp = decode_inputs(2, 16, 2, 128, ragged=(100, 3000), seed=31)
    pinp = prefill_inputs(1, 384, 16, 2, 128, seed=32)
    q, k, v = (to_gpu_bf16(dinp[x]) for x in ("q", "k", "v"))
    sl = to_gpu_i32(dinp["seqlens"])
    pq, pk, pv = (to_gpu_bf16(pinp[x]) for x in ("q", "k", "v"))
    say("graph capture: decode + prefill")

    o_ref, lse_ref = g.decode(q, k, v, sl, num_splits=4)
    po_ref, plse_ref = g.prefill_causal(pq, pk, pv)
    torch.cuda.synchronize()

    ws = g.decode_workspace(2, 16, 2, 128, k.shape[1], 4)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    po = torch.empty_like(po_ref)
    plse = torch.empty_like(plse_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.decode(q, k, v, sl, num_splits=4, out=o, lse=lse, workspace=ws)
        g.prefill_causal(pq, pk, pv, out=po, lse=plse)
    for r in range(3):
        for t in (o, lse, po, plse):
            t.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"decode replay {r}"
        assert torch.equal(po, po_ref) and torch.equal(plse, plse_ref), f"prefill replay {r}"
