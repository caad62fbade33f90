"""Chunked causal prefill over a paged KV cache on the GPU.

The paged kernel fetches every K/V tile page by page into the same on-chip layout as the
contiguous chunk kernel, so on the same keys the two must agree bit for bit; the contiguous
kernel is itself checked against the oracle (``test_gpu_prefill_chunk.py``), and one case
here is checked against the oracle directly.  Pool rows that hold no visible key are a bf16
NaN and table entries past the visible blocks are -1, so a kernel that read either would
show it.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads import LLAMA_PREFILL
from gqa_workloads.generate import BF16_QUIET_NAN, chunk_inputs, for_config
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def to_pages(x, keys, page, order, nb):
    """Rows [0, keys) of each sequence of x [B, S, H_kv, d] into a pool of pages at the
    positions order[b * nb + i]; every other pool row is NaN."""
    B, _, H_kv, d = x.shape
    pool = np.full((len(order), page, H_kv, d), BF16_QUIET_NAN, dtype=np.uint16)
    for b in range(B):
        for i in range(nb):
            rows = min(page, keys - i * page)
            pool[order[b * nb + i], :rows] = x[b, i * page:i * page + rows]
    return pool


def paged_case(inp, q_start, T, page, seed, spare=3, extra_cols=2):
    keys = q_start + T
    B = inp["k"].shape[0]
    nb = -(-keys // page)
    order = np.random.default_rng(seed).permutation(B * nb + spare).astype(np.int32)
    table = np.full((B, nb + extra_cols), -1, dtype=np.int32)
    for b in range(B):
        table[b, :nb] = order[b * nb:(b + 1) * nb]
    kp = to_pages(inp["k"], keys, page, order, nb)
    vp = to_pages(inp["v"], keys, page, order, nb)
    return kp, vp, table


def run_both(inp, q_start, T, page, seed):
    kp, vp, table = paged_case(inp, q_start, T, page, seed)
    q = to_gpu_bf16(inp["q"])
    keys = q_start + T
    k, v = (to_gpu_bf16(np.ascontiguousarray(inp[x][:, :keys])) for x in ("k", "v"))
    oc, lc = g.prefill_chunk(q, k, v, q_start=q_start)
    op, lp = g.prefill_chunk_paged(q, to_gpu_bf16(kp), to_gpu_bf16(vp), to_gpu_i32(table), q_start)
    torch.cuda.synchronize()
    return (oc, lc), (op, lp), (kp, vp, table)


CASES = [
    # (B, T, q_start, H_q, H_kv, page)
    (1, 256, 256, 8, 2, 16),       # whole q-block after one of context, pages of 16
    (1, 100, 37, 8, 2, 16),        # ragged start and end inside pages
    (2, 300, 1000, 16, 2, 48),     # pages of 48 (not a power of two), B = 2
    (1, 513, 2047, 8, 8, 32),      # three q-blocks, MHA, pages of 32
    (3, 40, 5, 16, 2, 16),         # short chunk near the start, B = 3
    (1, 1, 499, 8, 2, 64),         # a single query token
    (1, 17, 0, 4, 4, 16),          # q_start = 0: a whole short prompt
    (1, 700, 300, 64, 8, 256),     # Llama heads, pages of 256
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_paged_chunk_equals_contiguous(case, gpu_available):
    B, T, q_start, H_q, H_kv, page = case
    inp = chunk_inputs(B, T, q_start + T, H_q, H_kv, 128, seed=800 + T + q_start)
    say(f"paged prefill chunk {case}")
    (oc, lc), (op, lp), _ = run_both(inp, q_start, T, page, seed=801 + page)
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_paged_chunk_against_oracle(gpu_available):
    B, T, q_start, page = 2, 200, 333, 16
    inp = chunk_inputs(B, T, q_start + T, 16, 2, 128, seed=810)
    say("paged prefill chunk against the oracle")
    _, (op, lp), _ = run_both(inp, q_start, T, page, seed=811)
    o_ref, lse_ref = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"], q_start=q_start)
    say(f"  {check(to_f64(op), to_f64(lp), o_ref, lse_ref, 'paged chunk')}")


def test_paged_chunk_entry_outside_pool_reads_zeros(gpu_available):
    """A visible block whose table entry lies outside the pool reads as zero rows: the result
    is that of the contiguous kernel on a cache whose rows of that block are zero."""
    B, T, q_start, page = 2, 150, 100, 16
    inp = chunk_inputs(B, T, q_start + T, 8, 2, 128, seed=820)
    kp, vp, table = paged_case(inp, q_start, T, page, seed=821)
    bad = table.copy()
    bad[0, 3] = kp.shape[0] + 7
    bad[1, 0] = -5
    q = to_gpu_bf16(inp["q"])
    say("paged prefill chunk, table entries outside the pool")
    op, lp = g.prefill_chunk_paged(q, to_gpu_bf16(kp), to_gpu_bf16(vp), to_gpu_i32(bad), q_start)
    k, v = inp["k"][:, :q_start + T].copy(), inp["v"][:, :q_start + T].copy()
    for x in (k, v):
        x[0, 3 * page:4 * page] = 0
        x[1, 0:page] = 0
    oc, lc = g.prefill_chunk(q, to_gpu_bf16(k), to_gpu_bf16(v), q_start=q_start)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_paged_chunk_llama(gpu_available):
    """The last 2048 tokens of the Llama S = 8192 prompt as one chunk over pages of 16."""
    cfg = LLAMA_PREFILL
    full = for_config(cfg)
    T, q_start = 2048, cfg.S - 2048
    inp = {"q": full["q"][:, q_start:].copy(), "k": full["k"], "v": full["v"]}
    del full
    say(f"paged prefill chunk {cfg.name} T={T} q_start={q_start} pages of 16")
    (oc, lc), (op, lp), _ = run_both(inp, q_start, T, 16, seed=830)
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_paged_chunk_per_sequence_starts(gpu_available):
    """Each sequence's chunk at its own position (a device array of starts): every sequence
    of the batched call equals the call for that sequence alone, bit for bit; a start outside
    [0, table capacity - T_q] is clamped on the device, O is the clamped window's and the
    sequence's LSE is NaN."""
    B, T, page, keys = 3, 150, 16, 1150
    inp = chunk_inputs(B, T, keys, 16, 2, 128, seed=840)
    kp, vp, table = paged_case(inp, keys - T, T, page, seed=841)
    cap = table.shape[1] * page
    q = to_gpu_bf16(inp["q"])
    kpg, vpg, tbl = to_gpu_bf16(kp), to_gpu_bf16(vp), to_gpu_i32(table)
    for starts in ([0, 333, 1000], [-5, 17, 5000]):
        say(f"paged prefill chunk, per-sequence starts {starts}")
        ob, lb = g.prefill_chunk_paged(q, kpg, vpg, tbl, to_gpu_i32(np.array(starts, np.int32)))
        for b, s_raw in enumerate(starts):
            s = min(max(s_raw, 0), cap - T)
            o1, l1 = g.prefill_chunk_paged(q[b:b + 1].contiguous(), kpg, vpg,
                                           tbl[b:b + 1].contiguous(), s)
            torch.cuda.synchronize()
            # bit patterns: a clamped chunk may reach the pool's NaN rows, in both calls alike
            assert torch.equal(ob[b:b + 1].view(torch.int16), o1.view(torch.int16)), (starts, b)
            if s == s_raw:
                assert torch.equal(lb[b:b + 1].view(torch.int32), l1.view(torch.int32)), (starts, b)
            else:      # clamped: flagged by a NaN LSE on every row of the sequence
                assert torch.isnan(lb[b]).all(), (starts, b)
