"""Paged-cache decode (block-table gather, split-KV sweep, LSE merge) on the GPU.

Every case checks the GPU against the fp64 oracle (``oracle.decode_paged``:
gather through the block table, then the plain decode definition).  Pools are
filled with a bf16 NaN wherever no token lives and table entries past a
sequence's last block are -1, so a kernel that read either would show it.
The paged sweep does the same arithmetic in the same order as the unpaged one,
so with the same split plan the two must also agree bit for bit.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads import LLAMA_DECODE, LLAMA_RAGGED_DECODE
from gqa_workloads.generate import decode_inputs, paged_decode_inputs
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def upload(p):
    return (to_gpu_bf16(p["q"]), to_gpu_bf16(p["k_pool"]), to_gpu_bf16(p["v_pool"]),
            to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"]))


def run_paged(p, num_splits=0, use_seqlens=True):
    q, kp, vp, tbl, sl = upload(p)
    B, H_q, d = p["q"].shape
    ws = g.decode_workspace(B, H_q, p["k_pool"].shape[2], d, p["S_max"], num_splits)
    ws.fill_(0xFF)        # NaN in every slot: one read without being written shows
    o, lse = g.decode_paged(q, kp, vp, tbl, sl if use_seqlens else None, num_splits=num_splits,
                            workspace=ws)
    torch.cuda.synchronize()
    return o, lse


def oracle_paged(p, use_seqlens=True):
    sl = p["seqlens"] if use_seqlens else np.full(len(p["seqlens"]), p["S_max"], np.int32)
    return oracle.decode_paged(p["q"], p["k_pool"], p["v_pool"], p["block_table"], sl,
                               p["page_size"])


@pytest.mark.parametrize("page", [16, 128])
def test_paged_llama_ragged_batch_full(page, gpu_available):
    """The batched long-context Llama workload (B=8, lengths uniform on [4096, 131072])
    with its cache in pages of 16 (the common default) and 128 tokens."""
    cfg = LLAMA_RAGGED_DECODE
    p = paged_decode_inputs(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, page, seed=cfg.seed,
                            ragged=cfg.ragged)
    say(f"paged decode {cfg.name} page={page} seqlens={p['seqlens'].tolist()}")
    o, lse = run_paged(p, cfg.num_splits)
    o_ref, lse_ref = oracle_paged(p)
    say(f"  {check(to_f64(o), to_f64(lse), o_ref, lse_ref, f'{cfg.name} page {page}')}")


def test_paged_equals_unpaged_bitwise(gpu_available):
    """Same tokens, same split plan: the paged sweep reproduces the unpaged one exactly."""
    cfg = LLAMA_DECODE
    for page in (16, 64):
        p = paged_decode_inputs(1, cfg.H_q, cfg.H_kv, cfg.d, page, S_max=cfg.S_kv, seed=cfg.seed)
        u = decode_inputs(1, cfg.H_q, cfg.H_kv, cfg.d, S_max=cfg.S_kv, seed=cfg.seed)
        say(f"paged vs unpaged S={cfg.S_kv} page={page}")
        op, lp = run_paged(p, cfg.num_splits)
        q, k, v = (to_gpu_bf16(u[x]) for x in ("q", "k", "v"))
        ou, lu = g.decode(q, k, v, to_gpu_i32(u["seqlens"]), num_splits=cfg.num_splits)
        torch.cuda.synchronize()
        assert torch.equal(op, ou) and torch.equal(lp, lu)
    o_ref, lse_ref = oracle_paged(p)
    check(to_f64(op), to_f64(lp), o_ref, lse_ref, "paged llama s32768")


CASES = [
    # (B, H_q, H_kv, d, page, lengths (lo, hi) or fixed, num_splits)
    (3, 8, 2, 32, 16, (1, 700), 4),        # tiny group-of-4 heads, d = 32
    (2, 8, 1, 64, 32, (1, 2000), 0),       # MQA, d = 64
    (2, 16, 1, 128, 48, (100, 999), 3),    # page of 48: not a power of two
    (2, 32, 1, 32, 16, (257, 257), 2),     # G = 32: two head groups per KV head
    (2, 4, 4, 128, 272, (5000, 9000), 8),  # G = 1, pages of 272 tokens
    (4, 64, 8, 128, 16, (1, 40), 1),       # lengths below one slab, single chunk
    (1, 8, 2, 128, 16, (1, 1), 1),         # a single cached key
    (2, 24, 6, 64, 64, (3000, 5000), 0),   # 6 KV heads: 2 per workgroup, library splits
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_paged_shapes(case, gpu_available):
    B, H_q, H_kv, d, page, ragged, splits = case
    p = paged_decode_inputs(B, H_q, H_kv, d, page, seed=300 + sum(case[:5]), ragged=ragged)
    say(f"paged decode case {case} seqlens={p['seqlens'].tolist()}")
    o, lse = run_paged(p, splits)
    o_ref, lse_ref = oracle_paged(p)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, str(case))


def test_paged_without_seqlens_and_with_empty_sequence(gpu_available):
    p = paged_decode_inputs(3, 8, 2, 128, 32, S_max=320, seed=41)
    say("paged decode, no seqlens")
    o, lse = run_paged(p, 4, use_seqlens=False)
    o_ref, lse_ref = oracle_paged(p, use_seqlens=False)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "no seqlens")
    p["seqlens"] = np.array([0, 320, 33], dtype=np.int32)
    say("paged decode, an empty sequence")
    o, lse = run_paged(p, 4)
    o_ref, lse_ref = oracle_paged(p)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "empty")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_paged_shared_prefix_pages(gpu_available):
    """Sequences whose tables share leading pages (a common prompt) and one that reuses
    another's pages in a different order."""
    p = paged_decode_inputs(3, 16, 2, 128, 16, S_max=1024, seed=42)
    tbl = p["block_table"]
    tbl[1, :40] = tbl[0, :40]                 # first 640 tokens shared with sequence 0
    tbl[2] = tbl[0][::-1]                     # sequence 0's pages, reversed
    p["q"][1] = p["q"][0]
    p["seqlens"] = np.array([1024, 640, 1000], dtype=np.int32)
    say("paged decode, shared pages")
    o, lse = run_paged(p, 8)
    o_ref, lse_ref = oracle_paged(p)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "shared pages")
    # sequence 1 sees exactly sequence 0's first 640 tokens with the same queries
    p2 = dict(p)
    p2["seqlens"] = np.array([640, 640, 1000], dtype=np.int32)
    o2, lse2 = run_paged(p2, 8)
    assert torch.equal(o2[0], o[1]) and torch.equal(lse2[0], lse[1])


def test_paged_entry_outside_pool_reads_zeros(gpu_available):
    """A live table entry outside [0, num_pages) is not dereferenced: its tokens read as
    zero rows, which is what a page of zeros gives."""
    p = paged_decode_inputs(2, 8, 2, 128, 16, S_max=200, seed=43)
    bad = p["block_table"].copy()
    bad[0, 3] = p["k_pool"].shape[0] + 5
    bad[1, 0] = -7
    q, kp, vp, _, sl = upload(p)
    say("paged decode, table entries outside the pool")
    o, lse = g.decode_paged(q, kp, vp, to_gpu_i32(bad), sl, num_splits=2)
    torch.cuda.synchronize()
    # reference: the same table pointing at an extra all-zero page
    zp = dict(p)
    zero = p["k_pool"].shape[0]
    zp["k_pool"] = np.concatenate([p["k_pool"], np.zeros_like(p["k_pool"][:1])])
    zp["v_pool"] = np.concatenate([p["v_pool"], np.zeros_like(p["v_pool"][:1])])
    zt = p["block_table"].copy()
    zt[0, 3] = zero
    zt[1, 0] = zero
    zp["block_table"] = zt
    o_ref, lse_ref = oracle_paged(zp)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "entries outside the pool")


def test_paged_multi_token_decode(gpu_available):
    """T_q = 4 query tokens per sequence over a paged cache: against the oracle (the
    multi-token decode of the gathered caches) and bitwise against the unpaged kernel."""
    p = paged_decode_inputs(3, 16, 2, 128, 16, ragged=(2, 3000), seed=44)
    rng = np.random.default_rng(45)
    from gqa_workloads.generate import bf16_bits_from_f32
    q4 = bf16_bits_from_f32(rng.standard_normal((3, 4, 16, 128), dtype=np.float32))
    p["seqlens"][0] = 2                          # two tokens at negative positions
    q, kp, vp, tbl, sl = upload(p)
    qg = to_gpu_bf16(q4)
    say(f"paged multi-token decode seqlens={p['seqlens'].tolist()}")
    o, lse = g.decode_paged(qg, kp, vp, tbl, sl)
    k = oracle.gather_pages(p["k_pool"], p["block_table"], p["seqlens"], 16)
    v = oracle.gather_pages(p["v_pool"], p["block_table"], p["seqlens"], 16)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_tokens(q4, k, v, p["seqlens"])
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "paged T=4")
    ou, lu = g.decode_tokens(qg, to_gpu_bf16(k), to_gpu_bf16(v), sl)
    torch.cuda.synchronize()
    assert torch.equal(o, ou) and torch.equal(lse, lu)
