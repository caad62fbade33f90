"""Seeded synthetic inputs, as bf16 bit patterns in numpy uint16 arrays.

The same bytes feed the fp64 oracle (through ctypes) and the GPU (through a
torch upload), so both sides see identical inputs.  Values are N(0, 1) drawn in
float32 and rounded to bfloat16 with round-to-nearest-even done on the bit
pattern here, so the result does not depend on any library's conversion.

Each tensor draws from its own PCG64 stream spawned from the workload seed
(Q, K, V, lengths, outlier mask), so changing one shape does not shift another
tensor's values.

Layouts (row-major, innermost last):
  decode  q [B, H_q, d];      k, v [B, S_max, H_kv, d];  seqlens int32 [B]
  prefill q [B, S, H_q, d];   k, v [B, S, H_kv, d]
"""
import numpy as np

BF16_QUIET_NAN = np.uint16(0x7FC0)

_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_LEN, _STREAM_OUTLIER = range(5)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits.

    Inputs must be finite (the generator only produces finite normals).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(5)]


def _normal_bf16(rng, shape, chunk_rows: int = 1 << 22) -> np.ndarray:
    """N(0,1) bf16 bits of the given shape, drawn in row-major order in bounded chunks."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    pos = 0
    while pos < total:
        n = min(chunk_rows, total - pos)
        out[pos:pos + n] = bf16_bits_from_f32(rng.standard_normal(n, dtype=np.float32))
        pos += n
    return out.reshape(shape)


def decode_inputs(B, H_q, H_kv, d, S_max=None, seed=0, ragged=None, nan_fill=True):
    """Inputs of one decode launch.

    With ``ragged=(lo, hi)`` each sequence length is uniform on the inclusive
    range [lo, hi]; the cache is allocated to the longest one and the rows past
    each sequence's end hold a bf16 NaN pattern (``nan_fill``), so a kernel that
    read them would produce NaN.  Without ``ragged`` every length is ``S_max``.
    Returns a dict with q, k, v (uint16 bf16 bits), seqlens (int32) and S_max.
    """
    rq, rk, rv, rlen, _ = _streams(seed)
    if ragged is not None:
        lo, hi = ragged
        seqlens = rlen.integers(lo, hi, endpoint=True, size=B).astype(np.int32)
        S_max = int(seqlens.max())
    else:
        if S_max is None:
            raise ValueError("S_max is required without ragged lengths")
        seqlens = np.full(B, S_max, dtype=np.int32)
    q = _normal_bf16(rq, (B, H_q, d))
    k = np.empty((B, S_max, H_kv, d), dtype=np.uint16)
    v = np.empty((B, S_max, H_kv, d), dtype=np.uint16)
    for b in range(B):
        n = int(seqlens[b])
        k[b, :n] = _normal_bf16(rk, (n, H_kv, d))
        v[b, :n] = _normal_bf16(rv, (n, H_kv, d))
        if n < S_max:
            fill = BF16_QUIET_NAN if nan_fill else np.uint16(0)
            k[b, n:] = fill
            v[b, n:] = fill
    return {"q": q, "k": k, "v": v, "seqlens": seqlens, "S_max": S_max}


def prefill_inputs(B, S, H_q, H_kv, d, seed=0, outlier_frac=0.0, outlier_scale=1.0):
    """Inputs of one causal prefill launch.

    With ``outlier_frac > 0`` each key row (b, s, h_kv) is independently chosen
    with that probability and its whole d-vector is multiplied by
    ``outlier_scale`` after the bf16 rounding (a power-of-two scale keeps the
    values exact).  V is never scaled.  Returns q, k, v (uint16 bits) and the
    boolean outlier mask [B, S, H_kv].
    """
    rq, rk, rv, _, rout = _streams(seed)
    q = _normal_bf16(rq, (B, S, H_q, d))
    k = _normal_bf16(rk, (B, S, H_kv, d))
    v = _normal_bf16(rv, (B, S, H_kv, d))
    mask = np.zeros((B, S, H_kv), dtype=bool)
    if outlier_frac > 0.0:
        mask = rout.random((B, S, H_kv)) < outlier_frac
        scale = np.float32(outlier_scale)
        rows = k[mask]
        k[mask] = bf16_bits_from_f32(f32_from_bf16_bits(rows) * scale)
    return {"q": q, "k": k, "v": v, "outlier_mask": mask}


def for_config(cfg, nan_fill=True):
    """Inputs of a workload from ``gqa_workloads.CONFIGS``."""
    if cfg.kind == "decode":
        return decode_inputs(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, S_max=cfg.S_kv, seed=cfg.seed,
                             ragged=cfg.ragged, nan_fill=nan_fill)
    return prefill_inputs(cfg.B, cfg.S, cfg.H_q, cfg.H_kv, cfg.d, seed=cfg.seed,
                          outlier_frac=cfg.outlier_frac, outlier_scale=cfg.outlier_scale)
