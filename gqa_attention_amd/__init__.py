"""gqa_attention_amd -- grouped-query fused attention for MI355X (gfx950).

A thin ctypes binding of ``libgqa_attn.so`` (C ABI in ``include/gqa_attn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor dtypes/shapes, allocates outputs and the decode workspace
with torch, and passes raw device pointers plus torch's current HIP stream.
There is no fallback: if the library is missing the calls raise.

Entry points (names follow the C ABI):
  decode(q, k_cache, v_cache, seqlens=None, ...)      -> (o, lse)
  decode_partials(...) / decode_combine(...)           the two stages of decode
  lse_merge(part_m2, part_l, part_o, split_counts)     -> (o, lse)
  prefill_causal(q, k, v, ...)                         -> (o, lse)
"""
import ctypes
import math
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libgqa_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gqa_attn.h")

_lib = None


class GQAError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status, name, detail):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


def load_library(path=LIBRARY):
    """Load libgqa_attn.so and declare its C signatures (no GPU call is made)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gqa_attention_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ci, cf, cs = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.gqa_status_string.argtypes = [ci]
    L.gqa_status_string.restype = ctypes.c_char_p
    L.gqa_last_error.argtypes = []
    L.gqa_last_error.restype = ctypes.c_char_p
    L.gqa_version.argtypes = []
    L.gqa_version.restype = ctypes.c_char_p
    L.gqa_decode_plan.argtypes = [ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                  ctypes.POINTER(cs)]
    L.gqa_decode_plan.restype = ci
    L.gqa_attn_decode.argtypes = [vp, vp, vp, i32p, vp, f32p, ci, ci, ci, ci, ci, cf, ci, vp, cs, vp]
    L.gqa_attn_decode.restype = ci
    L.gqa_decode_partials.argtypes = [vp, vp, vp, i32p, ci, ci, ci, ci, ci, cf, ci, vp, cs, vp]
    L.gqa_decode_partials.restype = ci
    L.gqa_decode_combine.argtypes = [vp, f32p, ci, ci, ci, ci, ci, ci, vp, cs, vp]
    L.gqa_decode_combine.restype = ci
    L.gqa_attn_decode_paged.argtypes = [vp, vp, vp, i32p, i32p, vp, f32p, ci, ci, ci, ci, ci, ci,
                                        ci, ci, cf, ci, vp, cs, vp]
    L.gqa_attn_decode_paged.restype = ci
    L.gqa_decode_tokens_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci),
                                         ctypes.POINTER(ci), ctypes.POINTER(cs)]
    L.gqa_decode_tokens_plan.restype = ci
    L.gqa_attn_decode_tokens.argtypes = [vp, vp, vp, i32p, vp, f32p, ci, ci, ci, ci, ci, ci, cf,
                                         ci, vp, cs, vp]
    L.gqa_attn_decode_tokens.restype = ci
    L.gqa_lse_merge.argtypes = [f32p, f32p, f32p, i32p, ci, vp, f32p, ci, ci, ci, vp]
    L.gqa_lse_merge.restype = ci
    L.gqa_attn_prefill_causal.argtypes = [vp, vp, vp, vp, f32p, ci, ci, ci, ci, ci, cf, vp]
    L.gqa_attn_prefill_causal.restype = ci
    L.gqa_attn_prefill_chunk.argtypes = [vp, vp, vp, vp, f32p, ci, ci, ci, ci, ci, ci, ci, cf, vp]
    L.gqa_attn_prefill_chunk.restype = ci
    L.gqa_attn_prefill_chunk_paged.argtypes = [vp, vp, vp, i32p, i32p, vp, f32p, ci, ci, ci, ci, ci,
                                               ci, ci, ci, ci, cf, vp]
    L.gqa_attn_prefill_chunk_paged.restype = ci
    L.gqa_fp8_page_bytes.argtypes = [ci, ci, ci]
    L.gqa_fp8_page_bytes.restype = cs
    L.gqa_kv_quantize_fp8.argtypes = [vp, i32p, i32p, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    L.gqa_kv_quantize_fp8.restype = ci
    L.gqa_kv_dequantize_fp8.argtypes = [vp, i32p, i32p, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    L.gqa_kv_dequantize_fp8.restype = ci
    L.gqa_attn_decode_paged_fp8.argtypes = [vp, vp, vp, i32p, i32p, vp, f32p, ci, ci, ci, ci, ci,
                                            ci, ci, ci, cf, ci, vp, cs, vp]
    L.gqa_attn_decode_paged_fp8.restype = ci
    L.gqa_prefill_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    L.gqa_prefill_bwd_workspace_bytes.restype = cs
    L.gqa_attn_prefill_causal_bwd.argtypes = [vp, vp, vp, vp, f32p, vp, vp, vp, vp, ci, ci, ci, ci,
                                              ci, cf, vp, cs, vp]
    L.gqa_attn_prefill_causal_bwd.restype = ci
    L.gqa_attn_decode_noalloc.argtypes = [vp, vp, vp, i32p, vp, f32p, ci, ci, ci, ci, ci, cf, ci,
                                          vp]
    L.gqa_attn_decode_noalloc.restype = ci
    L.gqa_decode_noalloc_max_workspace.argtypes = []
    L.gqa_decode_noalloc_max_workspace.restype = cs
    L.gqa_device_info.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(ci), ctypes.c_char_p, cs]
    L.gqa_device_info.restype = ci
    L.gqa_stream_read_sink_bytes.argtypes = []
    L.gqa_stream_read_sink_bytes.restype = cs
    L.gqa_stream_read.argtypes = [vp, cs, vp, vp]
    L.gqa_stream_read.restype = ci
    L.gqa_mfma_rate_sink_bytes.argtypes = []
    L.gqa_mfma_rate_sink_bytes.restype = cs
    L.gqa_mfma_rate.argtypes = [vp, cs, ci, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.gqa_mfma_rate.restype = ci
    if path == LIBRARY:
        _lib = L
    return L


def header_functions(header=HEADER):
    """Names of the functions ``include/gqa_attn.h`` declares."""
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gqa_\w+)\s*\(", text, flags=re.M)))


def _check(rc):
    if rc != 0:
        L = load_library()
        raise GQAError(rc, L.gqa_status_string(rc).decode(), L.gqa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scale(d, softmax_scale):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def device_info(device=0):
    """Compute units, peak engine clock (kHz) and architecture name of a HIP device."""
    L = load_library()
    cus, khz = ctypes.c_int(), ctypes.c_int()
    arch = ctypes.create_string_buffer(64)
    _check(L.gqa_device_info(device, ctypes.byref(cus), ctypes.byref(khz), arch, 64))
    return {"compute_units": cus.value, "clock_khz": khz.value, "arch": arch.value.decode()}


def stream_read(buf, sink=None):
    """One launch of the library's plain streaming-read kernel over the bytes of a GPU
    tensor (the decode's bandwidth calibration); returns the sink tensor it may write."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    L = load_library()
    if sink is None:
        sink = torch.empty(L.gqa_stream_read_sink_bytes(), dtype=torch.uint8, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(L.gqa_stream_read(_ptr(buf), nbytes - nbytes % 16, _ptr(sink), _stream(buf.device)))
    return sink


def mfma_rate(ops, iters, sink=None):
    """One launch of the library's matrix-core rate kernel on the operand bits of a GPU
    tensor (the prefill's calibration: rounds of independent bf16 32x32x16 products, nothing
    else); returns (sink tensor, FLOP count of the launch)."""
    if not isinstance(ops, torch.Tensor) or not ops.is_cuda or not ops.is_contiguous():
        raise ValueError("ops must be a contiguous GPU tensor")
    L = load_library()
    if sink is None:
        sink = torch.empty(L.gqa_mfma_rate_sink_bytes() // 4, dtype=torch.float32,
                           device=ops.device)
    nbytes = ops.numel() * ops.element_size()
    flop = ctypes.c_double()
    _check(L.gqa_mfma_rate(_ptr(ops), nbytes - nbytes % 16, int(iters), _ptr(sink),
                           ctypes.byref(flop), _stream(ops.device)))
    return sink, flop.value


def decode_plan(B, H_q, H_kv, d, S_max, num_splits=0):
    """Split plan of a decode launch as a dict: partitions (of the batch's 16-key tiles,
    one workgroup each per head-group row), states (partial-state slots per query head)
    and workspace_bytes."""
    L = load_library()
    P, N = ctypes.c_int(), ctypes.c_int()
    ws = ctypes.c_size_t()
    _check(L.gqa_decode_plan(B, H_q, H_kv, d, S_max, num_splits, ctypes.byref(P),
                             ctypes.byref(N), ctypes.byref(ws)))
    return {"partitions": P.value, "states": N.value, "workspace_bytes": ws.value}


def decode_workspace(B, H_q, H_kv, d, S_max, num_splits=0, device="cuda"):
    """A workspace tensor sized for a decode launch."""
    ws = decode_plan(B, H_q, H_kv, d, S_max, num_splits)["workspace_bytes"]
    return torch.empty(ws, dtype=torch.uint8, device=device)


def _decode_shapes(q, k_cache, v_cache, seqlens):
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, H_q, d = q.shape
    Bk, S_max, H_kv, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
        if seqlens.shape[0] != B:
            raise ValueError("seqlens must have B entries")
    return B, H_q, H_kv, d, S_max


def decode(q, k_cache, v_cache, seqlens=None, softmax_scale=None, num_splits=0, out=None,
           lse=None, workspace=None):
    """Split-KV GQA decode: q [B,H_q,d], caches [B,S_max,H_kv,d] bf16 -> (o [B,H_q,d], lse [B,H_q])."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, k_cache, v_cache, seqlens)
    if workspace is None:
        workspace = decode_workspace(B, H_q, H_kv, d, S_max, num_splits, q.device)
    o = torch.empty((B, H_q, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, H_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(l), B, H_q, H_kv, d,
        S_max, _scale(d, softmax_scale), num_splits, _ptr(workspace), workspace.numel(),
        _stream(q.device)))
    return o, l


def decode_noalloc(q, k_cache, v_cache, seqlens=None, softmax_scale=None, num_splits=0, out=None,
                   lse=None):
    """decode() with the library's own device workspace (gqa_attn_decode_noalloc): no
    workspace argument; calls that overlap on one GPU race (see the header)."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, k_cache, v_cache, seqlens)
    o = torch.empty((B, H_q, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, H_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(l), B, H_q, H_kv, d,
        S_max, _scale(d, softmax_scale), num_splits, _stream(q.device)))
    return o, l


def decode_paged(q, k_pool, v_pool, block_table, seqlens=None, softmax_scale=None, num_splits=0,
                 out=None, lse=None, workspace=None):
    """Split-KV GQA decode over a paged cache: pools [num_pages,page,H_kv,d] bf16;
    block_table [B,max_blocks] int32.  q [B,H_q,d] (one token per sequence) -> (o [B,H_q,d],
    lse [B,H_q]), or q [B,T_q,H_q,d] (the last T_q positions) -> (o [B,T_q,H_q,d],
    lse [B,H_q,T_q])."""
    one = q.dim() == 3
    q4 = q.unsqueeze(1) if one else q
    _need(q4, "q", torch.bfloat16, 4)
    _need(k_pool, "k_pool", torch.bfloat16, 4)
    _need(v_pool, "v_pool", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    B, T, H_q, d = q4.shape
    num_pages, page, H_kv, dk = k_pool.shape
    if dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != B:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, pools {tuple(k_pool.shape)} / "
                         f"{tuple(v_pool.shape)}, block_table {tuple(block_table.shape)}")
    max_blocks = block_table.shape[1]
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
        if seqlens.shape[0] != B:
            raise ValueError("seqlens must have B entries")
    if workspace is None:
        nbytes = decode_tokens_plan(B, T, H_q, H_kv, d, max_blocks * page,
                                    num_splits)["workspace_bytes"]
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H_q) if one else (B, H_q, T), dtype=torch.float32, device=q.device)
    _check(load_library().gqa_attn_decode_paged(
        _ptr(q4), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seqlens), _ptr(out),
        _ptr(lse), B, T, H_q, H_kv, d, page, num_pages, max_blocks, _scale(d, softmax_scale),
        num_splits, _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out, lse


def decode_tokens_plan(B, T_q, H_q, H_kv, d, S_max, num_splits=0):
    """Split plan of a multi-token decode (see decode_plan)."""
    L = load_library()
    P, N = ctypes.c_int(), ctypes.c_int()
    ws = ctypes.c_size_t()
    _check(L.gqa_decode_tokens_plan(B, T_q, H_q, H_kv, d, S_max, num_splits, ctypes.byref(P),
                                    ctypes.byref(N), ctypes.byref(ws)))
    return {"partitions": P.value, "states": N.value, "workspace_bytes": ws.value}


def decode_tokens(q, k_cache, v_cache, seqlens=None, softmax_scale=None, num_splits=0, out=None,
                  lse=None, workspace=None):
    """Decode of T_q tokens per sequence (the last T_q cached positions, causal among them):
    q [B,T_q,H_q,d], caches [B,S_max,H_kv,d] bf16 -> (o [B,T_q,H_q,d], lse [B,H_q,T_q])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, T, H_q, d = q.shape
    Bk, S_max, H_kv, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, 1)
        if seqlens.shape[0] != B:
            raise ValueError("seqlens must have B entries")
    if workspace is None:
        nbytes = decode_tokens_plan(B, T, H_q, H_kv, d, S_max, num_splits)["workspace_bytes"]
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H_q, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_decode_tokens(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(l), B, T, H_q, H_kv,
        d, S_max, _scale(d, softmax_scale), num_splits, _ptr(workspace), workspace.numel(),
        _stream(q.device)))
    return o, l


def decode_partials(q, k_cache, v_cache, seqlens, workspace, softmax_scale=None, num_splits=0):
    """Stage 1 of decode: fill ``workspace`` with the partial (m2, l, O) of every chunk."""
    B, H_q, H_kv, d, S_max = _decode_shapes(q, k_cache, v_cache, seqlens)
    _check(load_library().gqa_decode_partials(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), B, H_q, H_kv, d, S_max,
        _scale(d, softmax_scale), num_splits, _ptr(workspace), workspace.numel(),
        _stream(q.device)))


def decode_combine(workspace, out, lse, H_kv, S_max, num_splits=0):
    """Stage 2 of decode: merge the workspace's partials into ``out`` and ``lse``."""
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    B, H_q, d = out.shape
    _check(load_library().gqa_decode_combine(
        _ptr(out), _ptr(lse), B, H_q, H_kv, d, S_max, num_splits, _ptr(workspace),
        workspace.numel(), _stream(out.device)))


def workspace_views(workspace, B, H_q, H_kv, d, S_max, num_splits=0):
    """Views of a decode workspace: (seg [B, 2] int32 -- first state slot and slot count of
    each sequence --, m2 [N, H_q], l [N, H_q] float32, o [N, H_q, d] bfloat16), N state
    slots."""
    N = decode_plan(B, H_q, H_kv, d, S_max, num_splits)["states"]
    a256 = lambda n: (n + 255) // 256 * 256
    off_m2 = a256(B * 2 * 4)
    off_l = off_m2 + a256(N * H_q * 4)
    off_o = off_l + a256(N * H_q * 4)
    f = workspace.view(torch.uint8)
    seg = f[:B * 2 * 4].view(torch.int32).view(B, 2)
    m2 = f[off_m2:off_m2 + N * H_q * 4].view(torch.float32).view(N, H_q)
    l = f[off_l:off_l + N * H_q * 4].view(torch.float32).view(N, H_q)
    o = f[off_o:off_o + N * H_q * d * 2].view(torch.bfloat16).view(N, H_q, d)
    return seg, m2, l, o


def lse_merge(part_m2, part_l, part_o, split_counts=None, out=None, lse=None):
    """Merge partial states: m2, l [B,H_q,P] fp32 (m2 in log2 units), o [B,H_q,P,d] fp32."""
    _need(part_m2, "part_m2", torch.float32, 3)
    _need(part_l, "part_l", torch.float32, 3)
    _need(part_o, "part_o", torch.float32, 4)
    B, H_q, P, d = part_o.shape
    if tuple(part_m2.shape) != (B, H_q, P) or tuple(part_l.shape) != (B, H_q, P):
        raise ValueError("partial shapes disagree")
    if split_counts is not None:
        _need(split_counts, "split_counts", torch.int32, 1)
    o = torch.empty((B, H_q, d), dtype=torch.bfloat16, device=part_o.device) if out is None else out
    l = torch.empty((B, H_q), dtype=torch.float32, device=part_o.device) if lse is None else lse
    _check(load_library().gqa_lse_merge(_ptr(part_m2), _ptr(part_l), _ptr(part_o),
                                        _ptr(split_counts), P, _ptr(o), _ptr(l), B, H_q, d,
                                        _stream(part_o.device)))
    return o, l


def prefill_causal(q, k, v, softmax_scale=None, out=None, lse=None):
    """Causal GQA prefill: q [B,S,H_q,d], k/v [B,S,H_kv,d] bf16 -> (o [B,S,H_q,d], lse [B,H_q,S])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, S, H_q, d = q.shape
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    H_kv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H_q, S), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_prefill_causal(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, S, H_q, H_kv, d,
        _scale(d, softmax_scale), _stream(q.device)))
    return o, l


def prefill_chunk(q, k_cache, v_cache, q_start=None, softmax_scale=None, out=None, lse=None):
    """Causal prefill of a chunk: q [B,T_q,H_q,d] are tokens q_start .. q_start+T_q-1 of
    sequences whose caches k/v [B,S_kv,H_kv,d] hold them; q_start defaults to S_kv - T_q
    (the chunk is the cache's last T_q tokens).  -> (o [B,T_q,H_q,d], lse [B,H_q,T_q])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, T, H_q, d = q.shape
    S_kv = k_cache.shape[1]
    if (k_cache.shape[0] != B or k_cache.shape[3] != d or
            tuple(v_cache.shape) != tuple(k_cache.shape)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k_cache.shape)}, "
                         f"v {tuple(v_cache.shape)}")
    H_kv = k_cache.shape[2]
    qs = S_kv - T if q_start is None else int(q_start)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H_q, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_prefill_chunk(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(l), B, T, qs, S_kv, H_q, H_kv, d,
        _scale(d, softmax_scale), _stream(q.device)))
    return o, l


def prefill_chunk_paged(q, k_pool, v_pool, block_table, q_start, softmax_scale=None, out=None,
                        lse=None):
    """Causal prefill of a chunk over a paged cache: q [B,T_q,H_q,d] are the tokens
    q_start.. of each sequence (q_start an int, or an int32 device tensor [B] of per-sequence
    starts); pools [num_pages,page,H_kv,d] bf16; block_table [B,max_blocks] int32 ->
    (o [B,T_q,H_q,d], lse [B,H_q,T_q])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_pool, "k_pool", torch.bfloat16, 4)
    _need(v_pool, "v_pool", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    B, T, H_q, d = q.shape
    num_pages, page, H_kv, dk = k_pool.shape
    if dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != B:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, pools {tuple(k_pool.shape)} / "
                         f"{tuple(v_pool.shape)}, block_table {tuple(block_table.shape)}")
    starts = None
    if torch.is_tensor(q_start):
        _need(q_start, "q_start", torch.int32, 1)
        if q_start.shape[0] != B:
            raise ValueError("q_start must have B entries")
        starts, q_start = q_start, 0
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H_q, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(load_library().gqa_attn_prefill_chunk_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(starts), _ptr(o), _ptr(l),
        B, T, int(q_start), H_q, H_kv, d, page, num_pages, block_table.shape[1],
        _scale(d, softmax_scale), _stream(q.device)))
    return o, l


def prefill_bwd_workspace_bytes(B, S, H_q, H_kv, d):
    """Workspace bytes of ``prefill_causal_bwd``: the per-row statistics (LSE in log2 units
    and D, 8 bytes per query row and head)."""
    n = load_library().gqa_prefill_bwd_workspace_bytes(B, S, H_q, H_kv, d)
    if n == 0:
        raise ValueError(f"invalid backward sizes B={B} S={S} H_q={H_q} H_kv={H_kv} d={d}")
    return n


def prefill_bwd_workspace(B, S, H_q, H_kv, d, device="cuda"):
    return torch.empty(prefill_bwd_workspace_bytes(B, S, H_q, H_kv, d), dtype=torch.uint8,
                       device=device)


def prefill_causal_bwd(q, k, v, o, lse, d_o, softmax_scale=None, workspace=None, out=None):
    """Backward of causal GQA prefill: from the forward's q, k, v, its o and lse and the
    output gradient d_o, returns (dq [B,S,H_q,d], dk [B,S,H_kv,d], dv [B,S,H_kv,d]) bf16.
    ``out`` may give the three output tensors."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _need(t, name, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, S, H_q, d = q.shape
    H_kv = k.shape[2]
    if (tuple(k.shape) != (B, S, H_kv, d) or tuple(v.shape) != tuple(k.shape) or
            tuple(o.shape) != tuple(q.shape) or tuple(d_o.shape) != tuple(q.shape) or
            tuple(lse.shape) != (B, H_q, S)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, o {tuple(o.shape)}, d_o {tuple(d_o.shape)}, "
                         f"lse {tuple(lse.shape)}")
    ws = prefill_bwd_workspace(B, S, H_q, H_kv, d, q.device) if workspace is None else workspace
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
    _check(load_library().gqa_attn_prefill_causal_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
        B, S, H_q, H_kv, d, _scale(d, softmax_scale), _ptr(ws), ws.numel(), _stream(q.device)))
    return dq, dk, dv


def fp8_page_bytes(page_size, H_kv, d):
    """Bytes of one FP8 page: page_size rows of H_kv*d E4M3 codes, then page_size fp32 scales."""
    return load_library().gqa_fp8_page_bytes(page_size, H_kv, d)


def kv_quantize_fp8(x, block_table, seqlens=None, pool=None, num_pages=None, page_size=16):
    """Quantise a bf16 cache x [B, S_max, H_kv, d] into the pages of an FP8 pool (uint8
    [num_pages, page bytes]) through block_table [B, max_blocks]; returns the pool."""
    _need(x, "x", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    B, S_max, H_kv, d = x.shape
    pb = fp8_page_bytes(page_size, H_kv, d)
    if pool is None:
        if num_pages is None:
            raise ValueError("give pool or num_pages")
        pool = torch.zeros((num_pages, pb), dtype=torch.uint8, device=x.device)
    if pool.dtype != torch.uint8 or pool.dim() != 2 or pool.shape[1] != pb or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous uint8 [num_pages, {pb}]")
    _check(load_library().gqa_kv_quantize_fp8(
        _ptr(x), _ptr(seqlens), _ptr(block_table), _ptr(pool), B, S_max, H_kv, d, page_size,
        pool.shape[0], block_table.shape[1], _stream(x.device)))
    return pool


def kv_dequantize_fp8(pool, block_table, S_max, H_kv, d, seqlens=None, page_size=16, out=None):
    """The live tokens of an FP8 pool (uint8 [num_pages, page bytes]) as a bf16 cache
    [B, S_max, H_kv, d] (``out``, else a new zero-filled tensor); returns it."""
    _need(block_table, "block_table", torch.int32, 2)
    B = block_table.shape[0]
    pb = fp8_page_bytes(page_size, H_kv, d)
    if pool.dtype != torch.uint8 or pool.dim() != 2 or pool.shape[1] != pb or not pool.is_contiguous():
        raise ValueError(f"pool must be contiguous uint8 [num_pages, {pb}]")
    x = torch.zeros((B, S_max, H_kv, d), dtype=torch.bfloat16, device=pool.device) if out is None else out
    _need(x, "out", torch.bfloat16, 4)
    _check(load_library().gqa_kv_dequantize_fp8(
        _ptr(pool), _ptr(seqlens), _ptr(block_table), _ptr(x), B, S_max, H_kv, d, page_size,
        pool.shape[0], block_table.shape[1], _stream(pool.device)))
    return x


def decode_paged_fp8(q, k_pool, v_pool, block_table, seqlens=None, page_size=16, H_kv=None,
                     softmax_scale=None, num_splits=0, out=None, lse=None, workspace=None):
    """Decode over FP8 pools (uint8 [num_pages, page bytes]); q [B, H_q, d] or
    [B, T_q, H_q, d] bf16.  H_kv is needed to read the page layout (default: H_q's KV heads
    from the page size).  Returns (o, lse) as ``decode_paged``."""
    _need(q, "q", torch.bfloat16, q.dim())
    _need(block_table, "block_table", torch.int32, 2)
    if q.dim() == 3:
        B, H_q, d = q.shape
        T = 1
    else:
        B, T, H_q, d = q.shape
    num_pages, pb = k_pool.shape
    if H_kv is None:
        H_kv = (pb - 4 * page_size) // (page_size * d)
    if fp8_page_bytes(page_size, H_kv, d) != pb or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError(f"pool shape {tuple(k_pool.shape)} is not pages of {page_size} rows "
                         f"of {H_kv}x{d}")
    max_blocks = block_table.shape[1]
    S_max = max_blocks * page_size
    if workspace is None:
        nbytes = (decode_plan(B, H_q, H_kv, d, S_max, num_splits) if T == 1 else
                  decode_tokens_plan(B, T, H_q, H_kv, d, S_max, num_splits))["workspace_bytes"]
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    l = (torch.empty((B, H_q) if T == 1 else (B, H_q, T), dtype=torch.float32, device=q.device)
         if lse is None else lse)
    _check(load_library().gqa_attn_decode_paged_fp8(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seqlens), _ptr(o), _ptr(l),
        B, T, H_q, H_kv, d, page_size, num_pages, max_blocks, _scale(d, softmax_scale),
        num_splits, _ptr(workspace), workspace.numel(), _stream(q.device)))
    return o, l
