"""gqa_attn_decode_noalloc (the decode with the library's own device workspace) against
gqa_attn_decode with a caller workspace, through the C ABI, on two calls in a row -- the
second with a smaller input, so it runs on the array the first call left behind -- and
against the fp64 oracle.  Also: a decode whose plan needs more than the array holds is
rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads import LLAMA_DECODE, LLAMA_RAGGED_DECODE
from gqa_workloads.generate import decode_inputs, for_config
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def _abi_decode(L, fn, q, k, v, sl, num_splits, ws=None):
    B, H_q, d = q.shape
    S_max, H_kv = k.shape[1], k.shape[2]
    o = torch.full((B, H_q, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H_q), float("nan"), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = [ptr(q), ptr(k), ptr(v), ptr(sl), ptr(o), ptr(lse), B, H_q, H_kv, d, S_max,
            1.0 / np.sqrt(d), num_splits]
    if ws is not None:
        args += [ptr(ws), ws.numel()]
    rc = fn(*args, stream)
    assert rc == 0, (L.gqa_status_string(rc), L.gqa_last_error())
    return o, lse


def _case(inp, num_splits, use_seqlens):
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    sl = to_gpu_i32(inp["seqlens"]) if use_seqlens else None
    return q, k, v, sl


def test_noalloc_matches_decode_two_calls(gpu_available):
    L = g.load_library()
    big = for_config(LLAMA_RAGGED_DECODE)                 # B = 8, lengths up to 131072
    small = for_config(LLAMA_DECODE)                      # B = 1, 32768 keys
    cases = [("ragged B=8", big, LLAMA_RAGGED_DECODE.num_splits, True),
             ("Llama S=32768", small, LLAMA_DECODE.num_splits, False)]
    for name, inp, ns, use_sl in cases:
        say(f"noalloc decode {name}")
        q, k, v, sl = _case(inp, ns, use_sl)
        B, H_q, d = q.shape
        plan = g.decode_plan(B, H_q, k.shape[2], d, k.shape[1], ns)
        assert plan["workspace_bytes"] <= L.gqa_decode_noalloc_max_workspace()
        ws = torch.full((plan["workspace_bytes"],), 0xFF, dtype=torch.uint8, device="cuda")
        o_ref, l_ref = _abi_decode(L, L.gqa_attn_decode, q, k, v, sl, ns, ws)
        o_na, l_na = _abi_decode(L, L.gqa_attn_decode_noalloc, q, k, v, sl, ns)
        torch.cuda.synchronize()
        # same plan, same kernels: bit for bit
        assert torch.equal(o_na.view(torch.int16), o_ref.view(torch.int16)), name
        assert torch.equal(l_na, l_ref), name
        o64, l64 = oracle.decode(inp["q"], inp["k"], inp["v"],
                                 inp["seqlens"] if use_sl else None)
        say(f"  {check(to_f64(o_na), to_f64(l_na), o64, l64, name)}")
        del q, k, v, sl, ws


def test_noalloc_rejects_oversized_plan(gpu_available):
    L = g.load_library()
    # the most partitions the plan allows gives states beyond 16 MiB (65535 slots x 64
    # heads x 520 bytes), whatever the cache length
    inp = decode_inputs(1, 64, 8, 128, S_max=64, seed=5)
    q, k, v, sl = _case(inp, 0, False)
    plan = g.decode_plan(1, 64, 8, 128, 64, 65535)
    assert plan["workspace_bytes"] > L.gqa_decode_noalloc_max_workspace()
    o = torch.empty((1, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.gqa_attn_decode_noalloc(p(q), p(k), p(v), None, p(o), p(lse), 1, 64, 8, 128, 64,
                                   1.0 / np.sqrt(128), 65535, stream)
    assert L.gqa_status_string(rc) == b"GQA_ERR_WORKSPACE"
    assert b"workspace" in L.gqa_last_error()
