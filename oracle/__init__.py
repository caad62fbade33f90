"""fp64 CPU oracle for grouped-query attention (ctypes front end of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its binding) never does, and this package never imports the product.

Every function takes bf16 inputs as numpy uint16 bit patterns (the layouts of
``gqa_workloads.generate``) and returns float64 results.  The arithmetic lives
in ``oracle.c``; the header of that file states the definitions and cites the
passages they follow.

Functions: decode, paged decode, multi-token decode, whole-prompt and chunked causal
prefill (all rows or selected rows), the partial state and merge of split-KV decode,
the backward of whole-prompt causal prefill (dQ per query row, dK and dV per key row of a
KV head, or all of them), and the FP8 (E4M3) paged KV cache: the format, per-token
quantisation into pages, and decode over the dequantised pages.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, special cases and a brute-force check built on
library routines) and by the planted-mistake checks in
``tests/test_oracle_mutants.py``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]

_lib = None


def build(source=SOURCE, output=LIBRARY, extra_flags=()):
    """Compile ``oracle.c`` with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(output + ".tmp", output)
    return output


def _bind(lib):
    u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    ci, cd, cl = ctypes.c_int, ctypes.c_double, ctypes.c_long
    lib.oracle_decode.argtypes = [u16p, u16p, u16p, ctypes.c_void_p, f64p, f64p,
                                  ci, ci, ci, ci, ci, cd, ci]
    lib.oracle_decode.restype = ci
    lib.oracle_prefill_causal_rows.argtypes = [u16p, u16p, u16p, f64p, f64p,
                                               ci, ci, ci, ci, ci, cd, i32p, cl, ci]
    lib.oracle_prefill_causal_rows.restype = ci
    lib.oracle_prefill_chunk_rows.argtypes = [u16p, u16p, u16p, f64p, f64p,
                                              ci, ci, ci, ci, ci, ci, ci, cd, i32p, cl, ci]
    lib.oracle_prefill_chunk_rows.restype = ci
    lib.oracle_decode_partial.argtypes = [u16p, u16p, u16p, f64p, f64p, f64p,
                                          ci, ci, ci, ci, ci, cd, ci, ci, ci]
    lib.oracle_decode_partial.restype = ci
    lib.oracle_merge_states.argtypes = [f64p, f64p, f64p, cl, ci, ci, f64p, f64p]
    lib.oracle_merge_states.restype = ci
    lib.oracle_prefill_causal_bwd_rows.argtypes = [u16p, u16p, u16p, u16p, ctypes.c_void_p, f64p,
                                                   f64p, f64p, ci, ci, ci, ci, ci, cd, i32p, cl,
                                                   ci]
    lib.oracle_prefill_causal_bwd_rows.restype = ci
    lib.oracle_prefill_causal_bwd_keys.argtypes = [u16p, u16p, u16p, u16p, f64p, f64p, f64p, f64p,
                                                   ci, ci, ci, ci, ci, cd, i32p, cl, ci]
    lib.oracle_prefill_causal_bwd_keys.restype = ci
    lib.oracle_e4m3_value.argtypes = [ci]
    lib.oracle_e4m3_value.restype = cd
    lib.oracle_e4m3_encode.argtypes = [cd]
    lib.oracle_e4m3_encode.restype = ci
    lib.oracle_e4m3_scale_exponent.argtypes = [cd]
    lib.oracle_e4m3_scale_exponent.restype = ci
    lib.oracle_quantize_fp8_rows.argtypes = [u16p, cl, ci,
                                             np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS"),
                                             np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")]
    lib.oracle_quantize_fp8_rows.restype = None
    return lib


def load(path=None):
    """Load the oracle library (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def default_threads():
    """Host threads the oracle uses: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when the environment sets it (a machine's share of its cores)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else n


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def decode(q, k, v, seqlens=None, tau=None, nthreads=0, lib=None):
    """Attention of one query token per (sequence, query head) over its cached keys.

    q [B, H_q, d]; k, v [B, S_max, H_kv, d] (uint16 bf16 bits); seqlens int32 [B] or None.
    ``tau`` defaults to 1/sqrt(d).  Returns (o [B, H_q, d], lse [B, H_q]) in float64.
    """
    lib = lib or load()
    B, H_q, d = q.shape
    _, S_max, H_kv, _ = k.shape
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    o = np.zeros((B, H_q, d), dtype=np.float64)
    lse = np.zeros((B, H_q), dtype=np.float64)
    sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
    rc = lib.oracle_decode(_u16(q), _u16(k), _u16(v),
                           None if sl is None else sl.ctypes.data_as(ctypes.c_void_p),
                           o, lse, B, H_q, H_kv, d, S_max, tau, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_decode rejected its arguments (code {rc})")
    return o, lse


def prefill_causal_rows(q, k, v, rows, tau=None, nthreads=0, lib=None):
    """Causal attention (key j visible to query i iff j <= i) on selected rows.

    q [B, S, H_q, d]; k, v [B, S, H_kv, d]; rows int array [n, 3] of (b, h, i).
    Returns (o [n, d], lse [n]) in float64.
    """
    lib = lib or load()
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
    n = rows.shape[0]
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_prefill_causal_rows(_u16(q), _u16(k), _u16(v), o, lse, B, S, H_q, H_kv, d,
                                        tau, rows, n, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_prefill_causal_rows rejected its arguments (code {rc})")
    return o, lse


def prefill_causal(q, k, v, tau=None, nthreads=0, lib=None):
    """Causal prefill on every row: returns (o [B, S, H_q, d], lse [B, H_q, S])."""
    B, S, H_q, d = q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H_q), np.arange(S), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    o, lse = prefill_causal_rows(q, k, v, rows, tau=tau, nthreads=nthreads, lib=lib)
    o = o.reshape(B, H_q, S, d).transpose(0, 2, 1, 3).copy()
    return o, lse.reshape(B, H_q, S)


def prefill_chunk_rows(q, k, v, rows, q_start=None, tau=None, nthreads=0, lib=None):
    """Causal attention of a chunk of T query rows against S_kv cached keys, on selected rows.

    q [B, T, H_q, d]; k, v [B, S_kv, H_kv, d]; rows int array [n, 3] of (b, h, i).
    Query row i is token q_start + i and sees keys j <= q_start + i; ``q_start``
    defaults to S_kv - T (the chunk is the last T tokens: bottom-right alignment).
    Returns (o [n, d], lse [n]) in float64.
    """
    lib = lib or load()
    B, T, H_q, d = q.shape
    S_kv, H_kv = k.shape[1], k.shape[2]
    q_start = S_kv - T if q_start is None else int(q_start)
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
    n = rows.shape[0]
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_prefill_chunk_rows(_u16(q), _u16(k), _u16(v), o, lse, B, T, q_start, S_kv,
                                       H_q, H_kv, d, tau, rows, n, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_prefill_chunk_rows rejected its arguments (code {rc})")
    return o, lse


def prefill_chunk(q, k, v, q_start=None, tau=None, nthreads=0, lib=None):
    """Chunked causal prefill on every row: returns (o [B, T, H_q, d], lse [B, H_q, T])."""
    B, T, H_q, d = q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H_q), np.arange(T), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    o, lse = prefill_chunk_rows(q, k, v, rows, q_start=q_start, tau=tau, nthreads=nthreads,
                                lib=lib)
    o = o.reshape(B, H_q, T, d).transpose(0, 2, 1, 3).copy()
    return o, lse.reshape(B, H_q, T)


def decode_tokens(q, k, v, seqlens=None, tau=None, nthreads=0, lib=None):
    """Decode of T query tokens per sequence, the last T of its cached keys: token i of
    sequence b sits at position L_b - T + i (L_b = seqlens[b], keys [0, L_b) cached) and
    sees keys j <= L_b - T + i -- the G query heads' T tokens are the G*T rows that the
    M-fold stacks (ADR-0060 sections 0.5.2 and 5.2).  Per sequence this is the causal
    chunk of ``prefill_chunk`` with q_start = L_b - T; a token whose position is negative
    (L_b < T) sees no key and gets O = 0, LSE = -inf.

    q [B, T, H_q, d]; k, v [B, S_max, H_kv, d]; seqlens int32 [B] or None (= S_max).
    Returns (o [B, T, H_q, d], lse [B, H_q, T]) in float64.
    """
    B, T, H_q, d = q.shape
    S_max = k.shape[1]
    lens = np.full(B, S_max) if seqlens is None else np.asarray(seqlens)
    o = np.zeros((B, T, H_q, d), dtype=np.float64)
    lse = np.full((B, H_q, T), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), S_max))
        first = max(T - L, 0)              # tokens before it have negative positions
        if first >= T:
            continue
        ob, lb = prefill_chunk(q[b:b + 1, first:], k[b:b + 1, :L], v[b:b + 1, :L],
                               q_start=L - T + first, tau=tau, nthreads=nthreads, lib=lib)
        o[b, first:] = ob[0]
        lse[b, :, first:] = lb[0]
    return o, lse


def gather_pages(pool, block_table, seqlens, page_size):
    """The cache of every sequence in logical token order, read out of a paged pool.

    pool [num_pages, page_size, H_kv, d]; block_table int32 [B, max_blocks];
    seqlens int32 [B].  Token t of sequence b is row t % page_size of page
    block_table[b, t // page_size] ("Attention Kernel lineage" (V07), section 16,
    logical-token-to-page map).  Returns [B, max_blocks * page_size, H_kv, d]
    with the rows past each sequence's length left zero.
    """
    B, max_blocks = block_table.shape
    out = np.zeros((B, max_blocks * page_size) + pool.shape[2:], dtype=pool.dtype)
    for b in range(B):
        t = np.arange(int(seqlens[b]))
        pages = block_table[b, t // page_size]
        if np.any((pages < 0) | (pages >= pool.shape[0])):
            raise ValueError(f"sequence {b}: a live block maps outside the pool")
        out[b, :t.size] = pool[pages, t % page_size]
    return out


def decode_paged(q, k_pool, v_pool, block_table, seqlens, page_size, tau=None, nthreads=0,
                 lib=None):
    """Decode over a paged K/V cache: gather each sequence's keys through its block
    table (``gather_pages``), then the plain decode definition.  Returns (o, lse)."""
    k = gather_pages(k_pool, block_table, seqlens, page_size)
    v = gather_pages(v_pool, block_table, seqlens, page_size)
    return decode(q, k, v, seqlens, tau=tau, nthreads=nthreads, lib=lib)


def decode_partial(q, k, v, j0, j1, tau=None, nthreads=0, lib=None):
    """Partial state (m, l, O unnormalised) of every decode row over keys [j0, j1)."""
    lib = lib or load()
    B, H_q, d = q.shape
    _, S_max, H_kv, _ = k.shape
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    m = np.zeros((B, H_q), dtype=np.float64)
    l = np.zeros((B, H_q), dtype=np.float64)
    o = np.zeros((B, H_q, d), dtype=np.float64)
    rc = lib.oracle_decode_partial(_u16(q), _u16(k), _u16(v), m, l, o, B, H_q, H_kv, d, S_max,
                                   tau, int(j0), int(j1), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_decode_partial rejected its arguments (code {rc})")
    return m, l, o


def merge_states(m, l, o, lib=None):
    """Merge partial states: m, l [R, P]; o [R, P, d] -> (o [R, d], lse [R])."""
    lib = lib or load()
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    R, P = m.shape
    d = o.shape[-1]
    o_out = np.zeros((R, d), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    lib.oracle_merge_states(m, l, o, R, P, d, o_out, lse)
    return o_out, lse


def prefill_causal_bwd_rows(q, k, v, do, rows, D=None, tau=None, nthreads=0, lib=None):
    """Backward of causal prefill, query side, on selected rows (b, h, i): the gradient
    dQ_i = tau sum_j P_ij (dP_ij - D_i) k_j with dP_ij = dO_i . v_j and D_i = sum_j P_ij dP_ij
    ("Attention Kernel lineage" (V07), section 6.1).  ``D`` [n] (optional) replaces the
    exact D_i: the method forms D_i = dO_i . O_i from the stored forward output (section
    6.2), so with a rounded O it differs slightly from the exact value.

    q, do [B, S, H_q, d]; k, v [B, S, H_kv, d] (uint16 bf16 bits); rows int [n, 3].
    Returns (dq [n, d], lse [n], D [n]) in float64.
    """
    lib = lib or load()
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
    n = rows.shape[0]
    dq = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    D_in = None if D is None else np.ascontiguousarray(D, dtype=np.float64).reshape(n)
    D = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_prefill_causal_bwd_rows(_u16(q), _u16(k), _u16(v), _u16(do),
                                            None if D_in is None else
                                            D_in.ctypes.data_as(ctypes.c_void_p), dq, lse, D,
                                            B, S, H_q, H_kv, d, tau, rows, n,
                                            nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_prefill_causal_bwd_rows rejected its arguments (code {rc})")
    return dq, lse, D


def prefill_causal_bwd_keys(q, k, v, do, lse, D, keys, tau=None, nthreads=0, lib=None):
    """Backward of causal prefill, key side, on selected key rows (b, g, j) of the KV heads:
    dK_j = tau sum_h sum_{i >= j} dS_ij q_i and dV_j = sum_h sum_{i >= j} P_ij dO_i over the
    G query heads h of KV head g, with P_ij = exp(s_ij - LSE_i) re-formed from each row's
    LSE (V07 section 6.4) and dS_ij = P_ij (dP_ij - D_i).

    lse, D [B, H_q, S] float64 for every row (``prefill_causal_bwd_rows``); keys int [n, 3].
    Returns (dk [n, d], dv [n, d]) in float64.
    """
    lib = lib or load()
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    tau = 1.0 / np.sqrt(d) if tau is None else float(tau)
    keys = np.ascontiguousarray(keys, dtype=np.int32).reshape(-1, 3)
    n = keys.shape[0]
    dk = np.zeros((n, d), dtype=np.float64)
    dv = np.zeros((n, d), dtype=np.float64)
    rc = lib.oracle_prefill_causal_bwd_keys(_u16(q), _u16(k), _u16(v), _u16(do),
                                            np.ascontiguousarray(lse, dtype=np.float64),
                                            np.ascontiguousarray(D, dtype=np.float64), dk, dv,
                                            B, S, H_q, H_kv, d, tau, keys, n,
                                            nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_prefill_causal_bwd_keys rejected its arguments (code {rc})")
    return dk, dv


def prefill_causal_bwd(q, k, v, do, o=None, tau=None, nthreads=0, lib=None):
    """Backward of causal prefill on every row and key.

    ``o`` [B, S, H_q, d] (optional, uint16 bf16 bits): a stored forward output; D_i is then
    dO_i . O_i from it (V07 section 6.2, as the method forms D) instead of the exact row-wise
    dot of P and dP.  Returns (dq [B, S, H_q, d], dk [B, S, H_kv, d], dv [B, S, H_kv, d],
    lse [B, H_q, S], D [B, H_q, S]) in float64.
    """
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    b, h, i = np.meshgrid(np.arange(B), np.arange(H_q), np.arange(S), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    D_in = None if o is None else stored_output_D(o, do).reshape(-1)   # rows in (b, h, i) order
    dq, lse, D = prefill_causal_bwd_rows(q, k, v, do, rows, D=D_in, tau=tau, nthreads=nthreads,
                                         lib=lib)
    lse = lse.reshape(B, H_q, S)
    D = D.reshape(B, H_q, S)
    b, g, j = np.meshgrid(np.arange(B), np.arange(H_kv), np.arange(S), indexing="ij")
    keys = np.stack([b.ravel(), g.ravel(), j.ravel()], axis=1)
    dk, dv = prefill_causal_bwd_keys(q, k, v, do, lse, D, keys, tau=tau, nthreads=nthreads,
                                     lib=lib)
    dq = dq.reshape(B, H_q, S, d).transpose(0, 2, 1, 3).copy()
    dk = dk.reshape(B, H_kv, S, d).transpose(0, 2, 1, 3).copy()
    dv = dv.reshape(B, H_kv, S, d).transpose(0, 2, 1, 3).copy()
    return dq, dk, dv, lse, D


def stored_output_D(o, do):
    """D [B, H_q, S] = dO_i . O_i of a stored bf16 output (V07 section 6.2), in float64
    (products of bf16 values are exact in float64)."""
    o64 = _f32_of_bits(o).astype(np.float64)
    do64 = _f32_of_bits(do).astype(np.float64)
    return np.einsum("bshd,bshd->bhs", o64, do64)


def _f32_of_bits(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ---------------------------------------------------------------------------------------
# FP8 KV cache ("Attention Kernel lineage" (V07), section 17.7): each page of a pool holds
# its page_size token rows of E4M3 codes ([page_size][H_kv][d] bytes) followed by the
# page_size per-token fp32 scales.  The arithmetic (E4M3 values, encoding, the scale of a
# row) is in oracle.c; the functions below only lay rows out in pages.

def e4m3_table(lib=None):
    """The value of every E4M3 code (float64 [256]; NaN for 0x7F and 0xFF)."""
    lib = lib or load()
    return np.array([lib.oracle_e4m3_value(c) for c in range(256)])


def quantize_fp8_rows(x, lib=None):
    """Quantise rows of bf16 values (uint16 bits, last axis = one row): returns (codes
    uint8, same shape; scales float32, one per row), each row with one power-of-two scale."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    width = x.shape[-1]
    rows = x.reshape(-1, width)
    codes = np.zeros(rows.shape, dtype=np.uint8)
    scales = np.zeros(rows.shape[0], dtype=np.float32)
    lib.oracle_quantize_fp8_rows(rows, rows.shape[0], width, codes, scales)
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def fp8_page_bytes(page_size, H_kv, d):
    """Bytes of one FP8 page: the codes of its rows, then one fp32 scale per row."""
    return page_size * H_kv * d + 4 * page_size


def quantize_to_pages(x, seqlens, block_table, page_size, num_pages, fill=0, lib=None):
    """The FP8 pool of a cache x [B, S_max, H_kv, d] (bf16 bits): token t < seqlens[b] of
    sequence b is quantised as one row (its H_kv * d values) into row t % page_size of page
    block_table[b, t // page_size] (V07 section 16, logical token to page).  Bytes of
    slots no live token maps to keep ``fill``.  Returns uint8 [num_pages, page bytes]."""
    B, S_max, H_kv, d = x.shape
    pb = fp8_page_bytes(page_size, H_kv, d)
    pool = np.full((num_pages, pb), fill, dtype=np.uint8)
    codes, scales = quantize_fp8_rows(x.reshape(B, S_max, H_kv * d), lib=lib)
    data = page_size * H_kv * d
    for b in range(B):
        for t in range(int(seqlens[b])):
            pg, r = int(block_table[b, t // page_size]), t % page_size
            pool[pg, r * H_kv * d:(r + 1) * H_kv * d] = codes[b, t]
            pool[pg, data + 4 * r:data + 4 * r + 4] = np.frombuffer(scales[b, t].tobytes(), np.uint8)
    return pool


def dequantize_pages(pool, page_size, H_kv, d, lib=None):
    """Every slot of an FP8 pool as bf16 bits [num_pages, page_size, H_kv, d]: code value
    times its row's scale.  With power-of-two scales the product is exactly a bfloat16;
    anything else raises."""
    table = e4m3_table(lib)
    n = pool.shape[0]
    data = page_size * H_kv * d
    codes = pool[:, :data].reshape(n, page_size, H_kv, d)
    scales = pool[:, data:data + 4 * page_size].copy().view(np.float32).reshape(n, page_size)
    vals = table[codes] * scales.astype(np.float64)[:, :, None, None]
    if np.isnan(vals).any():
        raise ValueError("NaN code in the pool")
    with np.errstate(over="ignore"):      # (an overflow fails the exactness check below)
        f32 = vals.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    back = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if not np.array_equal(back, vals):
        raise ValueError("a dequantised value is not exactly a bfloat16")
    return bits


def decode_paged_fp8(q, k_pool, v_pool, block_table, seqlens, page_size, tau=None, nthreads=0,
                     lib=None):
    """Decode (one or T_q tokens per sequence) over FP8 pools: the pools dequantised
    (exactly, as bf16) and then the paged decode definition."""
    H_kv = None
    d = q.shape[-1]
    data_plus = k_pool.shape[1]
    H_kv = (data_plus - 4 * page_size) // (page_size * d)
    kb = dequantize_pages(k_pool, page_size, H_kv, d, lib=lib)
    vb = dequantize_pages(v_pool, page_size, H_kv, d, lib=lib)
    if q.ndim == 4:
        k = gather_pages(kb, block_table, seqlens, page_size)
        v = gather_pages(vb, block_table, seqlens, page_size)
        return decode_tokens(q, k, v, seqlens, tau=tau, nthreads=nthreads, lib=lib)
    return decode_paged(q, kb, vb, block_table, seqlens, page_size, tau=tau, nthreads=nthreads,
                        lib=lib)
