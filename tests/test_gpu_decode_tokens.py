"""Multi-token decode (T_q tokens per sequence, the M-fold of G * T_q rows) on the GPU.

Every case checks the GPU against the fp64 oracle (``oracle.decode_tokens``: per
sequence, the causal chunk of its last T_q positions).  Cache rows past each
length hold a bf16 NaN, and the workspace is filled with NaN bytes before each
call, so a read of either would show.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads import LLAMA_RAGGED_DECODE
from gqa_workloads.generate import bf16_bits_from_f32, decode_inputs
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def tokens_inputs(B, T, H_q, H_kv, d, S_max=None, ragged=None, seed=0):
    inp = decode_inputs(B, H_q, H_kv, d, S_max=S_max, ragged=ragged, seed=seed)
    rng = np.random.default_rng(seed + 1)
    inp["q"] = bf16_bits_from_f32(rng.standard_normal((B, T, H_q, d), dtype=np.float32))
    return inp


def run_tokens(inp, num_splits=0, use_seqlens=True):
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    B, T, H_q, d = inp["q"].shape
    S_max, H_kv = inp["k"].shape[1], inp["k"].shape[2]
    ws = torch.empty(g.decode_tokens_plan(B, T, H_q, H_kv, d, S_max, num_splits)["workspace_bytes"],
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    sl = to_gpu_i32(inp["seqlens"]) if use_seqlens else None
    o, lse = g.decode_tokens(q, k, v, sl, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, T, H_q, H_kv, d, lengths (lo, hi) or fixed S, num_splits)
    (1, 2, 64, 8, 128, 32768, 32),         # Llama heads, 2 tokens: 16 rows per KV head
    (3, 3, 8, 2, 64, (1, 500), 0),         # lengths below T: leading tokens see nothing
    (2, 16, 8, 1, 32, (20, 300), 4),       # MQA, 128 rows per KV head: 8 row groups
    (5, 5, 16, 2, 128, (1000, 3000), 0),   # 40 rows per KV head, 4 waves per head
    (4, 4, 4, 4, 128, (200, 900), 2),      # MHA, 4 rows per KV head
    (2, 3, 6, 2, 128, (100, 900), 0),      # G = 3: 9 rows per KV head
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_tokens_shapes(case, gpu_available):
    B, T, H_q, H_kv, d, S, splits = case
    ragged = S if isinstance(S, tuple) else None
    inp = tokens_inputs(B, T, H_q, H_kv, d, S_max=None if ragged else S, ragged=ragged,
                        seed=700 + sum(case[:5]))
    say(f"decode tokens case {case} seqlens={inp['seqlens'].tolist()}")
    o, lse = run_tokens(inp, splits)
    o_ref, lse_ref = oracle.decode_tokens(inp["q"], inp["k"], inp["v"], inp["seqlens"])
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, str(case))


def test_decode_tokens_llama_ragged_t4(gpu_available):
    """The batched long-context Llama workload with 4 query tokens per sequence."""
    cfg = LLAMA_RAGGED_DECODE
    inp = tokens_inputs(cfg.B, 4, cfg.H_q, cfg.H_kv, cfg.d, ragged=cfg.ragged, seed=cfg.seed)
    say(f"decode tokens {cfg.name} T=4 seqlens={inp['seqlens'].tolist()}")
    o, lse = run_tokens(inp, cfg.num_splits)
    o_ref, lse_ref = oracle.decode_tokens(inp["q"], inp["k"], inp["v"], inp["seqlens"])
    say(f"  {check(to_f64(o), to_f64(lse), o_ref, lse_ref, 'ragged T=4')}")


def test_decode_tokens_one_token_is_decode(gpu_available):
    """T_q = 1 runs the one-token decode: the same plan, bitwise the same result."""
    inp = decode_inputs(3, 64, 8, 128, ragged=(100, 5000), seed=71)
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    sl = to_gpu_i32(inp["seqlens"])
    say("decode tokens T=1 vs decode")
    o1, l1 = g.decode(q, k, v, sl)
    o2, l2 = g.decode_tokens(q[:, None].contiguous(), k, v, sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[..., 0])


def test_decode_tokens_equals_prefill_chunk(gpu_available):
    """The same tokens through the chunked-prefill kernel agree within the tolerance."""
    inp = tokens_inputs(1, 8, 16, 2, 128, S_max=3000, seed=72)
    say("decode tokens vs prefill chunk")
    o, lse = run_tokens(inp, 0, use_seqlens=False)
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    oc, lc = g.prefill_chunk(q, k, v)
    torch.cuda.synchronize()
    check(to_f64(o), to_f64(lse), to_f64(oc), to_f64(lc), "tokens vs chunk")


def test_decode_tokens_sequences_shorter_than_t(gpu_available):
    """Lengths 0, 1 and 3 with T_q = 4: tokens at negative positions see no key."""
    inp = tokens_inputs(4, 4, 8, 2, 64, S_max=50, seed=73)
    inp["seqlens"] = np.array([0, 1, 3, 50], dtype=np.int32)
    say("decode tokens, sequences shorter than T")
    o, lse = run_tokens(inp, 0)
    o_ref, lse_ref = oracle.decode_tokens(inp["q"], inp["k"], inp["v"], inp["seqlens"])
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, "short sequences")
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(o[1, :3] == 0) and torch.all(torch.isneginf(lse[1, :, :3]))
