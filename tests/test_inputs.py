"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from gqa_workloads import LLAMA_RAGGED_DECODE, TINY_DECODE
from gqa_workloads.generate import (bf16_bits_from_f32, decode_inputs, f32_from_bf16_bits,
                                    for_config, prefill_inputs)


def test_bf16_rounding_matches_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 3.0e38, 1e-40], dtype=np.float32)])
    # ties: 1 + 2^-8 is exactly halfway between two bf16 values, rounds to even (1.0)
    halfway = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    x = np.concatenate([x, halfway])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert f32_from_bf16_bits(ours[-2:]).tolist() == [1.0, 1.0 + 2.0 ** -6]


def test_generator_is_deterministic_and_seeded():
    a = for_config(TINY_DECODE)
    b = for_config(TINY_DECODE)
    for key in ("q", "k", "v", "seqlens"):
        assert np.array_equal(a[key], b[key])
    c = decode_inputs(1, 8, 2, 32, S_max=512, seed=TINY_DECODE.seed + 1)
    assert not np.array_equal(a["q"], c["q"])
    x = f32_from_bf16_bits(a["k"]).astype(np.float64)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05


def test_ragged_lengths_and_nan_tail():
    inp = decode_inputs(8, 4, 2, 16, ragged=(5, 40), seed=3)
    sl = inp["seqlens"]
    assert sl.dtype == np.int32 and sl.min() >= 5 and sl.max() <= 40
    assert inp["S_max"] == sl.max()
    for b in range(8):
        tail = inp["k"][b, sl[b]:]
        assert np.all(tail == 0x7FC0)
        assert np.all(np.isfinite(f32_from_bf16_bits(inp["k"][b, :sl[b]])))


def test_ragged_config_length_range():
    lo, hi = LLAMA_RAGGED_DECODE.ragged
    assert (lo, hi) == (4096, 131072)
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(LLAMA_RAGGED_DECODE.seed).spawn(5)[3]))
    sl = rng.integers(lo, hi, endpoint=True, size=8)
    assert sl.min() >= lo and sl.max() <= hi


def test_outlier_keys_scaled_exactly():
    base = prefill_inputs(1, 4096, 2, 2, 16, seed=9)
    out = prefill_inputs(1, 4096, 2, 2, 16, seed=9, outlier_frac=0.01, outlier_scale=8.0)
    mask = out["outlier_mask"]
    frac = mask.mean()
    assert 0.005 < frac < 0.015
    kb = f32_from_bf16_bits(base["k"])
    ko = f32_from_bf16_bits(out["k"])
    assert np.array_equal(ko[mask], kb[mask] * 8.0)
    assert np.array_equal(ko[~mask], kb[~mask])
    assert np.array_equal(out["q"], base["q"]) and np.array_equal(out["v"], base["v"])
