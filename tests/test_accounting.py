"""Byte/FLOP accounting against the figures the pages print (CPU only)."""
import json
import os

import pytest

from gqa_workloads import CONFIGS, LLAMA_DECODE, LLAMA_LONG_PREFILL, LLAMA_PREFILL, TINY_DECODE
from gqa_workloads import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_accounting.json")))


def test_score_matrix_bytes_match_page_table():
    g = GOLDEN["score_matrix_bytes_fp16_single_head"]
    for (n, _label), expected in zip(g["rows"], g["bytes"]):
        assert acc.score_matrix_bytes(n, 2) == expected


def test_kv_bytes_per_context_match_capacity_arithmetic():
    g = GOLDEN["kv_bytes_per_context_per_kv_head_d32"]
    assert acc.kv_bytes_per_context_token(1, g["head_dim"]) == g["bytes"]
    cap = GOLDEN["smem_capacity_boundary"]
    assert cap["budget_bytes"] // acc.kv_bytes_per_context_token(1, 32) == cap["context_tokens"]
    ref = GOLDEN["smem_refusal_at_1820"]
    assert acc.kv_bytes(ref["context_tokens"], 1, 32) == ref["bytes"]
    assert ref["bytes"] > cap["budget_bytes"]


def test_gqa_cache_saving():
    g = GOLDEN["gqa_cache_saving"]
    mha = acc.kv_bytes(1000, g["H"], 128)
    gqa = acc.kv_bytes(1000, g["g"], 128)
    assert mha // gqa == g["saving"]


def test_workload_byte_and_flop_totals():
    # tiny decode: 512 tokens * 2 KV heads * 128 B = 131072 B of K+V
    assert acc.decode_kv_bytes([TINY_DECODE.S_kv], TINY_DECODE.H_kv, TINY_DECODE.d) == 131072
    assert acc.decode_flop([512], 8, 32) == 524288
    # Llama decode: 32768 tokens * 8 KV heads * 512 B = 128 MiB
    assert acc.decode_kv_bytes([LLAMA_DECODE.S_kv], 8, 128) == 134217728
    assert acc.prefill_causal_flop(1, LLAMA_PREFILL.S, 64, 128) == pytest.approx(1.0995e12, rel=1e-4)
    assert acc.prefill_causal_flop(1, LLAMA_LONG_PREFILL.S, 64, 128) == pytest.approx(7.0369e13,
                                                                                    rel=1e-4)
    # exact causal count = metric count * (S+1)/S
    S = LLAMA_PREFILL.S
    assert acc.prefill_causal_flop_exact(1, S, 64, 128) == pytest.approx(
        acc.prefill_causal_flop(1, S, 64, 128) * (S + 1) / S, rel=1e-12)
    assert len(CONFIGS) == 5


@pytest.mark.parametrize("S,B", [(8192, 64), (65536, 64), (4096, 128), (1024, 32)])
def test_causal_tile_count_matches_keep_ratio(S, B):
    # square tiles: n(n+1)/2 kept of n^2, i.e. ratio 1/2 + 1/(2n) = 1/2 + B_c/(2N)
    n = S // B
    kept = acc.causal_tiles_kept(S, B, B)
    assert kept == n * (n + 1) // 2
    assert kept / (n * n) == pytest.approx(acc.causal_keep_ratio(S, B), rel=1e-12)


def test_causal_tile_count_rectangular():
    # B_r = 128 rows, B_c = 64 keys: q-block r keeps keys up to its last row
    assert acc.causal_tiles_kept(256, 128, 64) == 2 + 4
    assert acc.causal_tiles_kept(200, 128, 64) == 2 + 4   # ragged last block: rows 128..199


def test_backward_flop_is_five_products():
    """Five causal S x S x d products per head: 2.5x the forward (two products)."""
    assert acc.prefill_causal_bwd_flop(1, 8192, 64, 128) == 2.5 * acc.prefill_causal_flop(1, 8192, 64, 128)
    assert acc.prefill_causal_bwd_flop(2, 10, 3, 4) == 2 * 5 * 10 * 10 * 4 * 3


def test_fp8_decode_bytes():
    """FP8 pages: one byte per cached value plus a 4-byte scale per token and pool."""
    assert acc.decode_kv_bytes_fp8([32768], 8, 128) == 2 * 32768 * (8 * 128 + 4)
    assert acc.decode_kv_bytes_fp8([32768], 8, 128) * 2 - acc.decode_kv_bytes([32768], 8, 128) == 2 * 2 * 32768 * 4
