"""Workload definitions for grouped-query attention: shapes, seeds and sizes.

This package is shared by the fp64 oracle side (``oracle/``, the tests) and the
GPU side (the binding, the tests, ``bench.py``).  It holds the configuration
table, the seeded input generator (``generate``) and the byte/FLOP accounting
(``accounting``).  It contains none of the attention arithmetic itself.

The five workloads are the Llama3-70B-shaped head layout (H_q=64, H_kv=8, G=8,
d=128; ADR-0060 "AHBM GQA Fused Attention", section 0 reference dimensions)
plus a tiny group-of-4 decode at d=32 (the TileFoundry showcase's GQA decode
layer: 8 query heads, 2 KV heads, head size 32).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

BASE_SEED = 20260101


@dataclass(frozen=True)
class DecodeConfig:
    """One decode launch: T_q = 1 query token per sequence."""
    name: str
    index: int
    B: int
    H_q: int
    H_kv: int
    d: int
    S_kv: Optional[int]              # fixed context length, or None when ragged
    ragged: Optional[Tuple[int, int]] = None   # inclusive [lo, hi] for per-sequence lengths
    num_splits: int = 0              # chunks of the longest sequence (0 = library's choice)
    kind: str = field(default="decode")

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index


@dataclass(frozen=True)
class PrefillConfig:
    """One causal prefill launch: T_q = S_kv = S, key j visible to query i iff j <= i."""
    name: str
    index: int
    B: int
    H_q: int
    H_kv: int
    d: int
    S: int
    outlier_frac: float = 0.0        # fraction of key rows scaled by outlier_scale
    outlier_scale: float = 1.0
    kind: str = field(default="prefill")

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index


TINY_DECODE = DecodeConfig("tiny_decode_g4_d32", 1, B=1, H_q=8, H_kv=2, d=32, S_kv=512,
                           num_splits=4)
LLAMA_DECODE = DecodeConfig("llama3_70b_decode_s32768", 2, B=1, H_q=64, H_kv=8, d=128,
                            S_kv=32768, num_splits=32)
LLAMA_RAGGED_DECODE = DecodeConfig("llama3_70b_batched_ragged_decode_b8", 3, B=8, H_q=64, H_kv=8,
                                   d=128, S_kv=None, ragged=(4096, 131072), num_splits=64)
LLAMA_PREFILL = PrefillConfig("llama3_70b_causal_prefill_s8192", 4, B=1, H_q=64, H_kv=8, d=128,
                              S=8192)
LLAMA_LONG_PREFILL = PrefillConfig("llama3_70b_causal_prefill_s65536_outliers", 5, B=1, H_q=64,
                                   H_kv=8, d=128, S=65536, outlier_frac=0.01, outlier_scale=8.0)

CONFIGS = (TINY_DECODE, LLAMA_DECODE, LLAMA_RAGGED_DECODE, LLAMA_PREFILL, LLAMA_LONG_PREFILL)
BY_NAME = {c.name: c for c in CONFIGS}
