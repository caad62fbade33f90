"""FP8 (E4M3) paged KV cache on the GPU ("Attention Kernel lineage" (V07), section 17.7).

* The quantiser (``gqa_kv_quantize_fp8``) against the oracle's per-token quantisation into
  pages: identical bytes, codes and scales, with the slots no token maps to untouched.
* The FP8 decode (``gqa_attn_decode_paged_fp8``) over the oracle's pools: against the
  oracle's decode over the dequantised pages, and -- since every dequantised value is a
  bfloat16 -- bit for bit against the bf16 paged decode over those dequantised pages.  The
  FP8 pools carry NaN codes (0x7F) in every slot no token maps to, so a read of one shows.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16, to_gpu_i32
from gqa_workloads import LLAMA_DECODE
from gqa_workloads.generate import bf16_bits_from_f32, paged_decode_inputs
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def logical_caches(p):
    """The contiguous caches [B, max_blocks * page, H_kv, d] that a paged input holds."""
    return tuple(oracle.gather_pages(p[x], p["block_table"], p["seqlens"], p["page_size"])
                 for x in ("k_pool", "v_pool"))


def oracle_pools(p, xk, xv, fill):
    n = p["k_pool"].shape[0]
    return tuple(oracle.quantize_to_pages(x, p["seqlens"], p["block_table"], p["page_size"], n,
                                          fill=fill) for x in (xk, xv))


def nan_poisoned(pool, p, H_kv, d):
    """A copy of an FP8 pool with NaN codes (0x7F) in every code slot no token maps to."""
    page = p["page_size"]
    out = pool.copy()
    live = np.zeros((pool.shape[0], page), dtype=bool)
    for b, n in enumerate(p["seqlens"]):
        for t in range(int(n)):
            live[p["block_table"][b, t // page], t % page] = True
    codes = out[:, :page * H_kv * d].reshape(pool.shape[0], page, H_kv * d)
    codes[~live] = 0x7F
    return out


QUANT_CASES = [
    # (B, H_kv, d, page, lengths)
    (3, 8, 128, 16, (1, 700)),     # Llama KV heads, ragged, pages of 16
    (2, 2, 64, 32, (30, 300)),     # d = 64, pages of 32
    (2, 1, 8, 48, (1, 100)),       # a row of 8 values (most lanes idle), pages of 48
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[str(c) for c in QUANT_CASES])
def test_quantize_matches_oracle(case, gpu_available):
    B, H_kv, d, page, ragged = case
    p = paged_decode_inputs(B, 8, H_kv, d, page, ragged=ragged, seed=700 + d + page,
                            nan_fill=False)
    xk, xv = logical_caches(p)
    # special rows: all zero, large (scale above one), tiny (scale near the bottom)
    rng = np.random.default_rng(701)
    xk[0, 0] = 0
    if p["seqlens"][0] > 2:
        xk[0, 1] = bf16_bits_from_f32(rng.standard_normal((H_kv, d)).astype(np.float32) * 3e4)
        xk[0, 2] = bf16_bits_from_f32(rng.standard_normal((H_kv, d)).astype(np.float32) * 1e-30)
    n = p["k_pool"].shape[0]
    pb = g.fp8_page_bytes(page, H_kv, d)
    assert pb == oracle.fp8_page_bytes(page, H_kv, d)
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    for name, x in (("k", xk), ("v", xv)):
        say(f"fp8 quantise {case} {name}")
        pool = torch.full((n, pb), 0xAB, dtype=torch.uint8, device="cuda")
        g.kv_quantize_fp8(to_gpu_bf16(x), tbl, sl, pool=pool, page_size=page)
        torch.cuda.synchronize()
        ref = oracle.quantize_to_pages(x, p["seqlens"], p["block_table"], page, n, fill=0xAB)
        got = pool.cpu().numpy()
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{name}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"


def fp8_decode_case(p, H_kv, d, num_splits, q=None):
    """FP8 decode over the oracle's pools against the oracle, and bitwise against the bf16
    paged decode over the dequantised pages."""
    xk, xv = logical_caches(p)
    kq, vq = oracle_pools(p, xk, xv, fill=0)
    kb = oracle.dequantize_pages(kq, p["page_size"], H_kv, d)
    vb = oracle.dequantize_pages(vq, p["page_size"], H_kv, d)
    q = p["q"] if q is None else q
    qg = to_gpu_bf16(q)
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    k8 = torch.from_numpy(nan_poisoned(kq, p, H_kv, d)).cuda()
    v8 = torch.from_numpy(nan_poisoned(vq, p, H_kv, d)).cuda()
    o8, l8 = g.decode_paged_fp8(qg, k8, v8, tbl, sl, page_size=p["page_size"], H_kv=H_kv,
                                num_splits=num_splits)
    ob, lb = g.decode_paged(qg, to_gpu_bf16(kb), to_gpu_bf16(vb), tbl, sl, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob) and torch.equal(l8, lb), "FP8 decode differs from bf16 on dequantised pages"
    o_ref, l_ref = oracle.decode_paged_fp8(q, kq, vq, p["block_table"], p["seqlens"],
                                           p["page_size"])
    return check(to_f64(o8), to_f64(l8), o_ref, l_ref, "fp8 decode")


DECODE_CASES = [
    # (B, H_q, H_kv, page, lengths, num_splits)
    (3, 16, 2, 16, (1, 900), 4),
    (2, 8, 1, 32, (200, 2000), 0),     # MQA
    (4, 64, 8, 16, (1, 40), 1),        # lengths below one tile, one chunk
    (2, 24, 6, 64, (3000, 5000), 0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_fp8_decode_shapes(case, gpu_available):
    B, H_q, H_kv, page, ragged, splits = case
    p = paged_decode_inputs(B, H_q, H_kv, 128, page, ragged=ragged, seed=710 + H_q + page,
                            nan_fill=False)
    say(f"fp8 decode {case} seqlens={p['seqlens'].tolist()}")
    say(f"  {fp8_decode_case(p, H_kv, 128, splits)}")


D64_CASES = [
    # (B, T_q, H_q, H_kv, page, lengths, num_splits), head size 64
    (3, 1, 16, 2, 16, (1, 1200), 4),
    (2, 1, 8, 1, 32, (300, 2500), 0),      # MQA
    (2, 1, 32, 1, 16, (100, 900), 2),      # G = 32: two workgroup rows per KV head
    (2, 3, 16, 4, 48, (2, 700), 0),        # T_q = 3 (G * T_q = 12 rows), pages of 48
]


@pytest.mark.parametrize("case", D64_CASES, ids=[str(c) for c in D64_CASES])
def test_fp8_decode_head_size_64(case, gpu_available):
    B, T, H_q, H_kv, page, ragged, splits = case
    p = paged_decode_inputs(B, H_q, H_kv, 64, page, ragged=ragged, seed=740 + H_q + page + T,
                            nan_fill=False)
    q = None
    if T > 1:
        rng = np.random.default_rng(741)
        q = bf16_bits_from_f32(rng.standard_normal((B, T, H_q, 64)).astype(np.float32))
    say(f"fp8 decode d=64 {case} seqlens={p['seqlens'].tolist()}")
    say(f"  {fp8_decode_case(p, H_kv, 64, splits, q=q)}")


def test_fp8_decode_llama_s32768(gpu_available):
    """The Llama3-70B decode (S_kv = 32768, 64 query heads, 8 KV heads, 32 splits) over
    FP8 pages of 16 tokens in permuted pool order."""
    cfg = LLAMA_DECODE
    p = paged_decode_inputs(1, cfg.H_q, cfg.H_kv, cfg.d, 16, S_max=cfg.S_kv, seed=cfg.seed,
                            nan_fill=False)
    say(f"fp8 decode {cfg.name}")
    say(f"  {fp8_decode_case(p, cfg.H_kv, cfg.d, cfg.num_splits)}")


def test_fp8_multi_token_decode(gpu_available):
    """T_q = 4 query tokens per sequence over FP8 pages (32 rows per KV head)."""
    p = paged_decode_inputs(3, 16, 2, 128, 16, ragged=(2, 3000), seed=720, nan_fill=False)
    p["seqlens"][0] = 2                           # two tokens at negative positions
    rng = np.random.default_rng(721)
    q4 = bf16_bits_from_f32(rng.standard_normal((3, 4, 16, 128)).astype(np.float32))
    say(f"fp8 multi-token decode seqlens={p['seqlens'].tolist()}")
    say(f"  {fp8_decode_case(p, 2, 128, 0, q=q4)}")


def test_fp8_gpu_quantised_pool_decodes(gpu_available):
    """The whole FP8 path on the GPU -- quantise, then decode -- equals the decode over the
    oracle's pools (the quantiser's bytes are the oracle's)."""
    p = paged_decode_inputs(2, 16, 2, 128, 16, ragged=(500, 1500), seed=730, nan_fill=False)
    xk, xv = logical_caches(p)
    n = p["k_pool"].shape[0]
    pb = g.fp8_page_bytes(16, 2, 128)
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    say("fp8 quantise then decode on the GPU")
    kg = g.kv_quantize_fp8(to_gpu_bf16(xk), tbl, sl, num_pages=n, page_size=16)
    vg = g.kv_quantize_fp8(to_gpu_bf16(xv), tbl, sl, num_pages=n, page_size=16)
    qg = to_gpu_bf16(p["q"])
    o1, l1 = g.decode_paged_fp8(qg, kg, vg, tbl, sl, page_size=16, H_kv=2)
    kq, vq = oracle_pools(p, xk, xv, fill=0)
    o2, l2 = g.decode_paged_fp8(qg, torch.from_numpy(kq).cuda(), torch.from_numpy(vq).cuda(), tbl,
                                sl, page_size=16, H_kv=2)
    torch.cuda.synchronize()
    assert kg.shape == (n, pb)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("case", QUANT_CASES, ids=[str(c) for c in QUANT_CASES])
def test_dequantize_matches_oracle(case, gpu_available):
    """The inverse of the quantiser: the oracle's pools, and the GPU quantiser's, read back as
    the oracle's dequantised cache, bit for bit, on every live row (dead rows untouched)."""
    B, H_kv, d, page, ragged = case
    p = paged_decode_inputs(B, 8, H_kv, d, page, ragged=ragged, seed=750 + d + page,
                            nan_fill=False)
    xk, _ = logical_caches(p)
    # special rows: all zero, large (scale above one), tiny (scale near the bottom)
    rng = np.random.default_rng(751)
    xk[0, 0] = 0
    if p["seqlens"][0] > 2:
        xk[0, 1] = bf16_bits_from_f32(rng.standard_normal((H_kv, d)).astype(np.float32) * 3e4)
        xk[0, 2] = bf16_bits_from_f32(rng.standard_normal((H_kv, d)).astype(np.float32) * 1e-30)
    n = p["k_pool"].shape[0]
    S_max = p["block_table"].shape[1] * page
    kq = oracle.quantize_to_pages(xk, p["seqlens"], p["block_table"], page, n, fill=0)
    ref = oracle.gather_pages(oracle.dequantize_pages(kq, page, H_kv, d), p["block_table"],
                              p["seqlens"], page)
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    say(f"fp8 dequantise {case}")
    for name, pool in (("oracle pool", torch.from_numpy(kq).cuda()),
                       ("gpu pool", g.kv_quantize_fp8(to_gpu_bf16(xk), tbl, sl, num_pages=n,
                                                      page_size=page))):
        out = torch.full((B, S_max, H_kv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        g.kv_dequantize_fp8(pool, tbl, S_max, H_kv, d, sl, page_size=page, out=out)
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        for b, ln in enumerate(p["seqlens"]):
            assert np.array_equal(got[b, :ln], ref[b, :ln]), f"{name}, sequence {b}"
            assert torch.isnan(out[b, ln:].float()).all(), f"{name}: a dead row was written"


def test_prefill_chunk_over_dequantised_fp8_cache(gpu_available):
    """The chunked prefill on an FP8 cache by composition: dequantise the pools, then run the
    chunk -- equal to the chunk over the oracle's dequantised cache."""
    B, H_q, H_kv, d, page, T = 2, 16, 2, 128, 16, 96
    p = paged_decode_inputs(B, H_q, H_kv, d, page, S_max=400, seed=760, nan_fill=False)
    xk, xv = logical_caches(p)
    n = p["k_pool"].shape[0]
    S_max = p["block_table"].shape[1] * page
    tbl, sl = to_gpu_i32(p["block_table"]), to_gpu_i32(p["seqlens"])
    kq, vq = oracle_pools(p, xk, xv, fill=0)
    say("chunked prefill over a dequantised FP8 cache")
    k = g.kv_dequantize_fp8(torch.from_numpy(kq).cuda(), tbl, S_max, H_kv, d, sl, page_size=page)
    v = g.kv_dequantize_fp8(torch.from_numpy(vq).cuda(), tbl, S_max, H_kv, d, sl, page_size=page)
    rng = np.random.default_rng(761)
    q = to_gpu_bf16(bf16_bits_from_f32(rng.standard_normal((B, T, H_q, d)).astype(np.float32)))
    o1, l1 = g.prefill_chunk(q, k[:, :400].contiguous(), v[:, :400].contiguous(), q_start=400 - T)
    kb = oracle.gather_pages(oracle.dequantize_pages(kq, page, H_kv, d), p["block_table"],
                             p["seqlens"], page)
    vb = oracle.gather_pages(oracle.dequantize_pages(vq, page, H_kv, d), p["block_table"],
                             p["seqlens"], page)
    o2, l2 = g.prefill_chunk(q, to_gpu_bf16(kb[:, :400]), to_gpu_bf16(vb[:, :400]), q_start=400 - T)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
