"""Every entry point captured in a HIP graph gives the eager results on every replay."""
import pytest
import torch

import gqa_attention_amd as g
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads.generate import (decode_inputs, paged_decode_inputs, prefill_bwd_inputs,
                                      prefill_inputs)

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


def test_graph_replays_match_eager_widened_paths(gpu_available):
    """Paged, multi-token and FP8 decode (with the quantiser in the graph), the chunked
    prefill over pages and the prefill backward, captured together: every replay equals the
    eager calls bit for bit."""
    B, H_q, H_kv, d, page = 2, 16, 2, 128, 16
    p = paged_decode_inputs(B, H_q, H_kv, d, page, ragged=(40, 700), seed=33)
    q, kp, vp = (to_gpu_bf16(p[x]) for x in ("q", "k_pool", "v_pool"))
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    S_max = p["block_table"].shape[1] * page
    c = decode_inputs(B, H_q, H_kv, d, ragged=(40, 700), seed=34)   # contiguous, NaN tails
    kc, vc = to_gpu_bf16(c["k"]), to_gpu_bf16(c["v"])
    csl = to_gpu_i32(c["seqlens"])
    Sc = c["S_max"]
    q3 = to_gpu_bf16(decode_inputs(B, 3 * H_q, H_kv, d, S_max=8, seed=35)["q"]).view(B, 3, H_q, d)
    nb = -(-Sc // page)                      # FP8 pages of the contiguous cache
    perm = torch.randperm(B * nb, generator=torch.Generator().manual_seed(36)).to(torch.int32)
    ftbl = perm.view(B, nb).cuda()
    first_pages = ftbl[:, 0].long()          # every sequence has at least 40 live tokens
    pinp = prefill_bwd_inputs(1, 200, 8, 2, 128, seed=37)
    pq, pk, pv, pdo = (to_gpu_bf16(pinp[x]) for x in ("q", "k", "v", "do"))
    # the prompt's last 80 tokens as a chunk over 16-token pages (13 pages, permuted)
    cq = pq[:, 120:].contiguous()
    pages = torch.randperm(13, generator=torch.Generator().manual_seed(38)).cuda()
    kpool = torch.zeros((13, page, 2, d), dtype=torch.bfloat16, device="cuda")
    vpool = torch.zeros_like(kpool)
    kpool.view(13 * page, 2, d)[:200] = pk[0]
    vpool.view(13 * page, 2, d)[:200] = pv[0]
    kpool, vpool = kpool[pages], vpool[pages]            # page i of the prompt -> slot
    ctbl = torch.argsort(pages).to(torch.int32).view(1, 13).contiguous()
    say("graph capture: paged, multi-token, FP8 decode, quantiser, prefill backward")

    def run(bufs):
        g.decode_paged(q, kp, vp, tbl, sl, num_splits=4, out=bufs["po"], lse=bufs["plse"],
                       workspace=bufs["ws_p"])
        g.decode_tokens(q3, kc, vc, csl, out=bufs["to"], lse=bufs["tlse"], workspace=bufs["ws_t"])
        g.kv_quantize_fp8(kc, ftbl, csl, pool=bufs["fk"], page_size=page)
        g.kv_quantize_fp8(vc, ftbl, csl, pool=bufs["fv"], page_size=page)
        g.decode_paged_fp8(q, bufs["fk"], bufs["fv"], ftbl, csl, page_size=page, H_kv=H_kv,
                           num_splits=3, out=bufs["fo"], lse=bufs["flse"], workspace=bufs["ws_f"])
        g.prefill_chunk_paged(cq, kpool, vpool, ctbl, 120, out=bufs["co"], lse=bufs["clse"])
        g.prefill_causal(pq, pk, pv, out=bufs["so"], lse=bufs["slse"])
        g.prefill_causal_bwd(pq, pk, pv, bufs["so"], bufs["slse"], pdo, workspace=bufs["ws_b"],
                             out=(bufs["dq"], bufs["dk"], bufs["dv"]))

    def buffers():
        pb = g.fp8_page_bytes(page, H_kv, d)
        return {
            "po": torch.empty_like(q), "plse": torch.empty((B, H_q), dtype=torch.float32, device="cuda"),
            "ws_p": g.decode_workspace(B, H_q, H_kv, d, S_max, 4),
            "to": torch.empty_like(q3), "tlse": torch.empty((B, H_q, 3), dtype=torch.float32, device="cuda"),
            "ws_t": torch.empty(g.decode_tokens_plan(B, 3, H_q, H_kv, d, Sc)["workspace_bytes"],
                                dtype=torch.uint8, device="cuda"),
            "fk": torch.empty((B * nb, pb), dtype=torch.uint8, device="cuda"),
            "fv": torch.empty((B * nb, pb), dtype=torch.uint8, device="cuda"),
            "fo": torch.empty_like(q), "flse": torch.empty((B, H_q), dtype=torch.float32, device="cuda"),
            "ws_f": g.decode_workspace(B, H_q, H_kv, d, nb * page, 3),
            "co": torch.empty_like(cq), "clse": torch.empty((1, 8, 80), dtype=torch.float32, device="cuda"),
            "so": torch.empty_like(pq), "slse": torch.empty((1, 8, 200), dtype=torch.float32, device="cuda"),
            "ws_b": g.prefill_bwd_workspace(1, 200, 8, 2, 128),
            "dq": torch.empty_like(pq), "dk": torch.empty_like(pk), "dv": torch.empty_like(pv),
        }

    ref = buffers()
    for t in ("fk", "fv"):
        ref[t].zero_()
    run(ref)
    torch.cuda.synchronize()
    cap = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap)
    outs = ("po", "plse", "to", "tlse", "fk", "fv", "fo", "flse", "co", "clse", "so", "slse", "dq",
            "dk", "dv")
    for r in range(3):
        for name in outs:                    # eager work between replays
            t = cap[name]
            if t.dtype == torch.uint8:
                # pages: the bytes no token owns keep what the eager run left; the first
                # codes and the first scale of each sequence's first page are spoilt
                t.copy_(ref[name])
                t[first_pages, :16] = 0xFF
                t[first_pages, page * H_kv * d:page * H_kv * d + 4] = 0xFF
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in outs:
            assert torch.equal(cap[name], ref[name]), f"{name}, replay {r}"
