"""Chunked causal prefill (T_q rows at positions q_start.., keys j <= q_start + i) on the GPU.

Every case checks the GPU against the fp64 oracle (``oracle.prefill_chunk``).
Cache rows past the chunk's last token hold a bf16 NaN: the kernel must never
read them (a NaN row, even with zero weight, would poison the output).
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import bf16_bits, say, to_gpu_bf16
from gqa_workloads import LLAMA_LONG_PREFILL, LLAMA_PREFILL
from gqa_workloads.generate import BF16_QUIET_NAN, chunk_inputs, for_config
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def poison_tail(inp, end):
    """Cache rows at or past `end` become NaN (never visible to the chunk)."""
    for x in ("k", "v"):
        inp[x][:, end:] = BF16_QUIET_NAN


def run_chunk(inp, q_start, scale=None):
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    o, lse = g.prefill_chunk(q, k, v, q_start=q_start, softmax_scale=scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


SMALL = [
    # (B, T, q_start, S_kv, H_q, H_kv)
    (1, 256, 256, 512, 8, 2),       # a whole q-block after one q-block of context
    (1, 100, 37, 200, 8, 2),        # start not on a 32-key step, ragged, NaN tail
    (1, 64, 16, 80, 8, 1),          # each wave's diagonal spans two 32-key steps (MQA)
    (2, 300, 1000, 1300, 16, 2),    # bottom-right, B = 2, XCD remap active
    (1, 1, 499, 500, 8, 2),         # a single query token (decode through the prefill path)
    (1, 17, 0, 17, 4, 4),           # q_start = 0, T = S_kv: plain causal prefill (MHA)
    (1, 513, 2047, 2600, 8, 8),     # three q-blocks, ragged, odd start, NaN tail
    (3, 40, 5, 45, 16, 2),          # short chunk near the start, B = 3
    (1, 150, 70, 250, 6, 2),        # G = 3, start not on a 32-key step, NaN tail
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_chunk_small_full(case, gpu_available):
    B, T, q_start, S_kv, H_q, H_kv = case
    inp = chunk_inputs(B, T, S_kv, H_q, H_kv, 128, seed=500 + T + q_start)
    poison_tail(inp, q_start + T)
    say(f"prefill chunk {case}")
    _, _, _, o, lse = run_chunk(inp, q_start)
    o_ref, lse_ref = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"], q_start=q_start)
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, str(case))
    if q_start == 0:      # row 0 attends to key 0 only: O is V_0 exactly
        G = H_q // H_kv
        assert np.array_equal(bf16_bits(o[:, 0]), np.repeat(inp["v"][:, 0], G, axis=1))


def test_chunk_default_start_is_bottom_right(gpu_available):
    inp = chunk_inputs(1, 200, 650, 8, 2, 128, seed=61)
    say("prefill chunk, default q_start")
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    o1, l1 = g.prefill_chunk(q, k, v)
    o2, l2 = g.prefill_chunk(q, k, v, q_start=450)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"])
    check(to_f64(o1), to_f64(l1), o_ref, lse_ref, "default start")


def test_chunks_cover_whole_prompt(gpu_available):
    """Chunks run one after another over a prompt give the whole-prompt rows (within the
    tolerance of both against the oracle)."""
    S, H_q, H_kv = 1100, 16, 2
    inp = chunk_inputs(1, S, S, H_q, H_kv, 128, seed=62)
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    say("prefill chunks vs whole prompt")
    o_full, l_full = g.prefill_causal(q, k, v)
    o_ref, lse_ref = oracle.prefill_causal(inp["q"], inp["k"], inp["v"])
    check(to_f64(o_full), to_f64(l_full), o_ref, lse_ref, "whole")
    for a, b in ((0, 256), (256, 700), (700, 701), (701, S)):
        oc, lc = g.prefill_chunk(q[:, a:b].contiguous(), k[:, :b].contiguous(),
                                 v[:, :b].contiguous())
        torch.cuda.synchronize()
        check(to_f64(oc), to_f64(lc), o_ref[:, a:b], lse_ref[..., a:b], f"chunk [{a}, {b})")


def sample_chunk_rows(T, q_start, H_q, B, rng, n_random):
    rows = set()
    heads = sorted({0, H_q - 1, *rng.integers(0, H_q, size=6).tolist()})
    edges = [i for qb in range(0, T, 1024)
             for i in (qb - 1, qb, qb + 31, qb + 32, qb + 63, qb + 64, qb + 255, qb + 256)
             if 0 <= i < T]
    fixed = list(range(0, 16)) + list(range(max(T - 16, 0), T)) + edges
    for b in range(B):
        for h in heads:
            for i in fixed:
                rows.add((b, h, int(i)))
    for _ in range(n_random):
        rows.add((int(rng.integers(0, B)), int(rng.integers(0, H_q)), int(rng.integers(0, T))))
    return np.array(sorted(rows), dtype=np.int32)


def check_chunk_sampled(inp, q_start, o, lse, rows, what):
    o_ref, lse_ref = oracle.prefill_chunk_rows(inp["q"], inp["k"], inp["v"], rows,
                                               q_start=q_start)
    b, h, i = (torch.from_numpy(rows[:, c].astype(np.int64)).to(o.device) for c in range(3))
    return check(to_f64(o[b, i, h]), to_f64(lse[b, h, i]), o_ref, lse_ref, what)


@pytest.mark.parametrize("cfg,T", [(LLAMA_PREFILL, 2048), (LLAMA_LONG_PREFILL, 4096)],
                         ids=["s8192_last2048", "s65536_outliers_last4096"])
def test_chunk_llama_sampled(cfg, T, gpu_available):
    """The last T tokens of the Llama prompts as one chunk against the whole cache."""
    full = for_config(cfg)
    q_start = cfg.S - T
    inp = {"q": full["q"][:, q_start:].copy(), "k": full["k"], "v": full["v"]}
    del full
    say(f"prefill chunk {cfg.name} T={T} q_start={q_start}")
    _, _, _, o, lse = run_chunk(inp, q_start)
    rows = sample_chunk_rows(T, q_start, cfg.H_q, cfg.B, np.random.default_rng(63), 192)
    stats = check_chunk_sampled(inp, q_start, o, lse, rows, f"{cfg.name} chunk {T}")
    say(f"  {len(rows)} rows: {stats}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
