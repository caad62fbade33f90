"""Seeded synthetic inputs, as bf16 bit patterns in numpy uint16 arrays.

The same bytes feed the fp64 oracle (through ctypes) and the GPU (through a
torch upload), so both sides see identical inputs.  Values are N(0, 1) drawn in
float32 and rounded to bfloat16 with round-to-nearest-even done on the bit
pattern here, so the result does not depend on any library's conversion.

Each tensor draws from its own PCG64 stream spawned from the workload seed
(Q, K, V, lengths, outlier mask, pages, output gradient), so changing one shape does not shift another
tensor's values.

Layouts (row-major, innermost last):
  decode  q [B, H_q, d];      k, v [B, S_max, H_kv, d];  seqlens int32 [B]
  paged   q [B, H_q, d];      k_pool, v_pool [num_pages, page_size, H_kv, d];
          block_table int32 [B, max_blocks];  seqlens int32 [B]
  prefill q [B, S, H_q, d];   k, v [B, S, H_kv, d]
  chunk   q [B, T, H_q, d];   k, v [B, S_kv, H_kv, d]
  bwd     prefill inputs and dO [B, S, H_q, d] (the gradient of the output)
"""
import numpy as np

BF16_QUIET_NAN = np.uint16(0x7FC0)

_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_LEN, _STREAM_OUTLIER, _STREAM_PAGES, _STREAM_DOUT = \
    range(7)


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
    # child i of the seed sequence depends only on i, so adding streams shifts none
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(7)]


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
    rq, rk, rv, rlen = _streams(seed)[:4]
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


def paged_decode_inputs(B, H_q, H_kv, d, page_size, S_max=None, seed=0, ragged=None,
                        spare_pages=3, nan_fill=True):
    """Inputs of one decode launch over a paged K/V cache.

    Lengths, Q and the K/V rows of every sequence are the same values that
    ``decode_inputs`` draws for the same arguments; the rows are then scattered
    into pages of ``page_size`` tokens (token t of sequence b goes to row
    t % page_size of page block_table[b, t // page_size]) placed at randomly
    permuted positions of a pool that also holds ``spare_pages`` pages no table
    references.  Pool rows that hold no token carry a bf16 NaN (``nan_fill``),
    and table entries past a sequence's last block are -1, so a kernel that read
    either would show it.  Returns q, k_pool, v_pool, block_table, seqlens,
    page_size and S_max (= max_blocks * page_size, the table's key capacity).
    """
    rq, rk, rv, rlen = _streams(seed)[:4]
    rpage = _streams(seed)[_STREAM_PAGES]
    if ragged is not None:
        lo, hi = ragged
        seqlens = rlen.integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    else:
        if S_max is None:
            raise ValueError("S_max is required without ragged lengths")
        seqlens = np.full(B, S_max, dtype=np.int32)
    blocks = [-(-int(n) // page_size) for n in seqlens]
    max_blocks = max(max(blocks), 1)
    num_pages = sum(blocks) + spare_pages
    order = rpage.permutation(num_pages).astype(np.int32)
    fill = BF16_QUIET_NAN if nan_fill else np.uint16(0)
    q = _normal_bf16(rq, (B, H_q, d))
    k_pool = np.full((num_pages, page_size, H_kv, d), fill, dtype=np.uint16)
    v_pool = np.full((num_pages, page_size, H_kv, d), fill, dtype=np.uint16)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    used = 0
    for b in range(B):
        n = int(seqlens[b])
        kb = _normal_bf16(rk, (n, H_kv, d))
        vb = _normal_bf16(rv, (n, H_kv, d))
        for i in range(blocks[b]):
            page = int(order[used])
            used += 1
            table[b, i] = page
            rows = min(page_size, n - i * page_size)
            k_pool[page, :rows] = kb[i * page_size:i * page_size + rows]
            v_pool[page, :rows] = vb[i * page_size:i * page_size + rows]
    return {"q": q, "k_pool": k_pool, "v_pool": v_pool, "block_table": table,
            "seqlens": seqlens, "page_size": page_size, "S_max": max_blocks * page_size}


def chunk_inputs(B, T, S_kv, H_q, H_kv, d, seed=0):
    """Inputs of one chunked-prefill launch: T query rows against S_kv cached keys."""
    rq, rk, rv = _streams(seed)[:3]
    q = _normal_bf16(rq, (B, T, H_q, d))
    k = _normal_bf16(rk, (B, S_kv, H_kv, d))
    v = _normal_bf16(rv, (B, S_kv, H_kv, d))
    return {"q": q, "k": k, "v": v}


def prefill_inputs(B, S, H_q, H_kv, d, seed=0, outlier_frac=0.0, outlier_scale=1.0):
    """Inputs of one causal prefill launch.

    With ``outlier_frac > 0`` each key row (b, s, h_kv) is independently chosen
    with that probability and its whole d-vector is multiplied by
    ``outlier_scale`` after the bf16 rounding (a power-of-two scale keeps the
    values exact).  V is never scaled.  Returns q, k, v (uint16 bits) and the
    boolean outlier mask [B, S, H_kv].
    """
    rq, rk, rv, _, rout = _streams(seed)[:5]
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


def prefill_bwd_inputs(B, S, H_q, H_kv, d, seed=0, outlier_frac=0.0, outlier_scale=1.0):
    """Inputs of one backward launch of causal prefill: the forward's q, k, v (the same
    bytes as ``prefill_inputs`` with the same arguments) and the output gradient
    dO [B, S, H_q, d], N(0, 1) in bf16 from a stream of its own."""
    p = prefill_inputs(B, S, H_q, H_kv, d, seed=seed, outlier_frac=outlier_frac,
                       outlier_scale=outlier_scale)
    p["do"] = _normal_bf16(_streams(seed)[_STREAM_DOUT], (B, S, H_q, d))
    return p


def for_config(cfg, nan_fill=True):
    """Inputs of a workload from ``gqa_workloads.CONFIGS``."""
    if cfg.kind == "decode":
        return decode_inputs(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, S_max=cfg.S_kv, seed=cfg.seed,
                             ragged=cfg.ragged, nan_fill=nan_fill)
    return prefill_inputs(cfg.B, cfg.S, cfg.H_q, cfg.H_kv, cfg.d, seed=cfg.seed,
                          outlier_frac=cfg.outlier_frac, outlier_scale=cfg.outlier_scale)
