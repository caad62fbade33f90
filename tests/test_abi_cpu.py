"""The C ABI on the CPU: symbols, plans and argument checks (no kernel is launched).

Every call below fails validation on the host, before the library touches the
GPU, so these run without one.  Pointers are fake but aligned addresses that
are never dereferenced.
"""
import ctypes
import subprocess

import pytest

import gqa_attention_amd as g

OK, NULLP, SHAPE, UNSUP, SPLITS, WS, ALIGN, SCALE, HIP = range(9)
A = ctypes.c_void_p(0x10000)          # aligned fake device address
MIS = ctypes.c_void_p(0x10002)        # 2-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return g.load_library()


def test_library_exports_every_declared_function(lib):
    declared = g.header_functions()
    assert {"gqa_attn_decode", "gqa_attn_decode_paged", "gqa_attn_prefill_causal",
            "gqa_attn_prefill_chunk", "gqa_attn_decode_tokens", "gqa_decode_tokens_plan",
            "gqa_lse_merge", "gqa_decode_plan",
            "gqa_decode_partials", "gqa_decode_combine", "gqa_status_string",
            "gqa_last_error", "gqa_version"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in declared if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for f in declared:
        getattr(lib, f)


def test_status_strings(lib):
    names = [lib.gqa_status_string(i).decode() for i in range(9)]
    assert names == ["GQA_OK", "GQA_ERR_NULL_POINTER", "GQA_ERR_BAD_SHAPE", "GQA_ERR_UNSUPPORTED",
                     "GQA_ERR_SPLITS", "GQA_ERR_WORKSPACE", "GQA_ERR_ALIGNMENT", "GQA_ERR_SCALE",
                     "GQA_ERR_HIP"]
    assert lib.gqa_status_string(99).decode() == "GQA_ERR_UNKNOWN"
    assert b"gfx950" in lib.gqa_version()


@pytest.mark.parametrize("args,expect", [
    # (B, H_q, H_kv, d, S_max, num_splits) -> partitions (workgroups per head-group row)
    ((1, 64, 8, 128, 32768, 32), 256),     # Llama decode: 8 heads per workgroup, 256 partitions
    ((1, 64, 8, 128, 32768, 0), 256),      # auto: one workgroup per CU
    ((8, 64, 8, 128, 131072, 64), 256),    # ragged decode: the same 256, whatever the lengths
    ((1, 64, 8, 128, 32768, 1000), 1000),  # num_splits above the fill count is kept
    ((1, 8, 2, 32, 512, 4), 256),          # tiny decode: most partitions empty
    ((1, 32, 1, 32, 257, 2), 256),         # G = 32: one wave folds both 16-column blocks
    ((1, 48, 1, 32, 257, 2), 128),         # G = 48: two workgroup rows of 32 columns
    ((1, 24, 6, 64, 1000, 1), 86),         # 6 KV heads: 2 per workgroup, 3 rows
])
def test_decode_plan(args, expect):
    plan = g.decode_plan(*args)
    assert plan["partitions"] == expect
    B, H_q, _, d, _, _ = args
    assert plan["states"] == expect + B - 1
    a256 = lambda n: (n + 255) // 256 * 256
    n = plan["states"] * H_q
    assert plan["workspace_bytes"] == a256(B * 8) + 2 * a256(n * 4) + a256(n * d * 2)


def test_decode_plan_workspace_size_at_llama_shape():
    # 256 partitions x 64 heads x (m, l fp32; 128-wide O bf16) partial states, plus the
    # slot table
    plan = g.decode_plan(1, 64, 8, 128, 32768, 32)
    assert plan["workspace_bytes"] == 256 + 256 * 64 * (2 * 4 + 128 * 2)


@pytest.mark.parametrize("args,code", [
    ((1, 64, 7, 128, 1024, 0), SHAPE),       # H_kv does not divide H_q
    ((0, 64, 8, 128, 1024, 0), SHAPE),
    ((1, 64, 8, 128, 0, 0), SHAPE),
    ((1, 64, 8, 96, 1024, 0), UNSUP),        # head size without a kernel
    ((1, 64, 8, 128, 1024, -1), SPLITS),
    ((1, 64, 8, 128, 1024, 70000), SPLITS),
    ((8193, 8, 2, 32, 16, 0), SHAPE),        # batch above the LDS sequence table
    ((4096, 8, 2, 32, 1 << 30, 0), SHAPE),   # B * ceil(S_max / 16) >= 2^31
])
def test_decode_plan_rejects(lib, args, code):
    rc = lib.gqa_decode_plan(*args, None, None, None)
    assert rc == code
    assert lib.gqa_last_error().decode() != ""


def _decode(lib, q=A, k=A, v=A, seqlens=None, o=A, lse=A, B=1, H_q=8, H_kv=2, d=32, S=512,
            scale=0.17, splits=4, ws=A, ws_bytes=1 << 30):
    return lib.gqa_attn_decode(q, k, v, seqlens, o, lse, B, H_q, H_kv, d, S, scale, splits, ws,
                               ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(k=None), NULLP), (dict(v=None), NULLP), (dict(o=None), NULLP),
    (dict(lse=None), NULLP), (dict(ws=None), WS),
    (dict(q=MIS), ALIGN), (dict(o=MIS), ALIGN), (dict(seqlens=ctypes.c_void_p(0x10001)), ALIGN),
    (dict(ws=ctypes.c_void_p(0x10010)), WS),      # workspace not 256-byte aligned
    (dict(ws_bytes=100), WS),
    (dict(scale=-1.0), SCALE), (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE),
    (dict(H_kv=3), SHAPE), (dict(d=16), UNSUP), (dict(splits=-2), SPLITS),
])
def test_decode_rejects_before_launch(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_stage_calls_reject_before_launch(lib):
    assert lib.gqa_decode_partials(None, A, A, None, 1, 8, 2, 32, 512, 0.1, 4, A, 1 << 30,
                                   None) == NULLP
    assert lib.gqa_decode_combine(A, A, 1, 8, 2, 32, 512, 4, A, 10, None) == WS
    assert lib.gqa_decode_combine(MIS, A, 1, 8, 2, 32, 512, 4, A, 1 << 30, None) == ALIGN


def _paged(lib, q=A, kp=A, vp=A, tbl=A, seqlens=None, o=A, lse=A, B=1, T=1, H_q=8, H_kv=2,
           d=32, page=16, num_pages=64, max_blocks=32, scale=0.17, splits=4, ws=A,
           ws_bytes=1 << 30):
    return lib.gqa_attn_decode_paged(q, kp, vp, tbl, seqlens, o, lse, B, T, H_q, H_kv, d, page,
                                     num_pages, max_blocks, scale, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(tbl=None), NULLP), (dict(kp=None), NULLP), (dict(vp=MIS), ALIGN),
    (dict(tbl=ctypes.c_void_p(0x10002)), ALIGN),
    (dict(page=8), SHAPE), (dict(page=40), SHAPE), (dict(page=0), SHAPE),
    (dict(page=1 << 17), SHAPE),
    (dict(num_pages=0), SHAPE), (dict(max_blocks=0), SHAPE),
    (dict(num_pages=1 << 27, page=32), SHAPE),     # num_pages * page_size overflows 31 bits
    (dict(ws_bytes=100), WS), (dict(d=96), UNSUP), (dict(H_kv=3), SHAPE),
    (dict(scale=float("nan")), SCALE), (dict(T=0), SHAPE), (dict(T=17), SHAPE),
])
def test_paged_decode_rejects_before_launch(lib, kw, code):
    assert _paged(lib, **kw) == code
    assert lib.gqa_last_error().decode() != ""


@pytest.mark.parametrize("T,code", [(0, SHAPE), (17, SHAPE), (-1, SHAPE)])
def test_decode_tokens_rejects_token_count(lib, T, code):
    assert lib.gqa_decode_tokens_plan(1, T, 8, 2, 32, 512, 0, None, None, None) == code
    assert lib.gqa_attn_decode_tokens(A, A, A, None, A, A, 1, T, 8, 2, 32, 512, 0.1, 0, A,
                                      1 << 30, None) == code


def test_decode_tokens_plan_folds_rows():
    # 8 heads x 4 tokens = 32 rows per KV head: one wave folds both 16-column blocks
    p4 = g.decode_tokens_plan(1, 4, 64, 8, 128, 32768, 0)
    assert p4["partitions"] == 256 and p4["states"] == 256
    # 8 heads x 8 tokens = 64 rows: two workgroup rows of 32, so 128 partitions per row
    p8 = g.decode_tokens_plan(1, 8, 64, 8, 128, 32768, 0)
    assert p8["partitions"] == 128
    a256 = lambda n: (n + 255) // 256 * 256
    n = 256 * 64 * 4
    assert p4["workspace_bytes"] == 256 + 2 * a256(n * 4) + a256(n * 128 * 2)
    assert g.decode_tokens_plan(2, 1, 64, 8, 128, 1000, 0) == g.decode_plan(2, 64, 8, 128, 1000, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(m2=None), NULLP), (dict(o=MIS), ALIGN), (dict(P=0), SPLITS), (dict(P=70000), SPLITS),
    (dict(po=ctypes.c_void_p(0x10004)), ALIGN),
    (dict(d=48), UNSUP), (dict(B=0), SHAPE), (dict(counts=ctypes.c_void_p(0x10003)), ALIGN),
])
def test_lse_merge_rejects_before_launch(lib, kw, code):
    a = dict(m2=A, l=A, po=A, counts=None, P=4, o=A, lse=A, B=1, H_q=8, d=32)
    a.update(kw)
    assert lib.gqa_lse_merge(a["m2"], a["l"], a["po"], a["counts"], a["P"], a["o"], a["lse"],
                             a["B"], a["H_q"], a["d"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(lse=None), NULLP), (dict(k=MIS), ALIGN),
    (dict(H_kv=5), SHAPE), (dict(S=0), SHAPE), (dict(d=64), UNSUP), (dict(scale=-0.5), SCALE),
])
def test_prefill_rejects_before_launch(lib, kw, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, B=1, S=256, H_q=8, H_kv=2, d=128, scale=0.088)
    a.update(kw)
    assert lib.gqa_attn_prefill_causal(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["S"],
                                       a["H_q"], a["H_kv"], a["d"], a["scale"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(o=MIS), ALIGN), (dict(T=0), SHAPE), (dict(S=0), SHAPE),
    (dict(q_start=-1), SHAPE), (dict(q_start=200), SHAPE),     # q_start + T_q > S_kv
    (dict(T=300, q_start=0), SHAPE), (dict(H_kv=3), SHAPE), (dict(d=64), UNSUP),
    (dict(scale=float("inf")), SCALE),
])
def test_prefill_chunk_rejects_before_launch(lib, kw, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, B=1, T=100, q_start=150, S=256, H_q=8, H_kv=2, d=128,
             scale=0.088)
    a.update(kw)
    assert lib.gqa_attn_prefill_chunk(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"],
                                      a["q_start"], a["S"], a["H_q"], a["H_kv"], a["d"],
                                      a["scale"], None) == code
    assert lib.gqa_last_error().decode() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), SHAPE), (dict(q_start=-1), SHAPE), (dict(page=24), SHAPE), (dict(page=0), SHAPE),
    (dict(num_pages=0), SHAPE), (dict(max_blocks=15), SHAPE), (dict(tbl=None), NULLP),
    (dict(tbl=ctypes.c_void_p(0x10002)), ALIGN), (dict(d=64), UNSUP), (dict(H_kv=3), SHAPE),
    (dict(q=MIS), ALIGN), (dict(scale=-1.0), SCALE), (dict(qs=ctypes.c_void_p(0x10002)), ALIGN),
    # 8193 blocks of 16 keys: past the table row the kernel stages on chip
    (dict(T=1, q_start=8192 * 16, max_blocks=9000), UNSUP),
])
def test_prefill_chunk_paged_rejects_before_launch(lib, kw, code):
    a = dict(q=A, k=A, v=A, tbl=A, qs=None, o=A, lse=A, B=1, T=100, q_start=150, H_q=8, H_kv=2,
             d=128, page=16, num_pages=64, max_blocks=16, scale=0.088)
    a.update(kw)
    assert lib.gqa_attn_prefill_chunk_paged(a["q"], a["k"], a["v"], a["tbl"], a["qs"], a["o"],
                                            a["lse"],
                                            a["B"], a["T"], a["q_start"], a["H_q"], a["H_kv"],
                                            a["d"], a["page"], a["num_pages"], a["max_blocks"],
                                            a["scale"], None) == code
    assert lib.gqa_last_error().decode() != ""


def test_prefill_bwd_workspace_size(lib):
    """Statistics only, [B, H_q, ceil(S/64), 128] fp32 (dK and dV are summed over the query
    heads on chip); 0 for invalid sizes."""
    B, S, H_q, H_kv, d = 2, 300, 8, 2, 128
    assert lib.gqa_prefill_bwd_workspace_bytes(B, S, H_q, H_kv, d) == B * H_q * 5 * 128 * 4
    for bad in ((0, S, H_q, H_kv, d), (B, 0, H_q, H_kv, d), (B, S, H_q, 3, d), (B, S, H_q, H_kv, 64)):
        assert lib.gqa_prefill_bwd_workspace_bytes(*bad) == 0


BWD_WS = 1 << 30


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(dk=None), NULLP), (dict(lse=None), NULLP), (dict(do=MIS), ALIGN),
    (dict(lse=ctypes.c_void_p(0x10002)), ALIGN), (dict(dv=MIS), ALIGN), (dict(H_kv=3), SHAPE),
    (dict(S=0), SHAPE), (dict(B=0), SHAPE), (dict(d=64), UNSUP), (dict(scale=float("nan")), SCALE),
    (dict(ws=None), WS), (dict(ws=ctypes.c_void_p(0x10010)), WS), (dict(ws_bytes=4096), WS),
])
def test_prefill_bwd_rejects_before_launch(lib, kw, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, B=1, S=256, H_q=8, H_kv=2, d=128,
             scale=0.088, ws=A, ws_bytes=BWD_WS)
    a.update(kw)
    assert lib.gqa_attn_prefill_causal_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                                           a["dq"], a["dk"], a["dv"], a["B"], a["S"], a["H_q"],
                                           a["H_kv"], a["d"], a["scale"], a["ws"], a["ws_bytes"],
                                           None) == code
    assert lib.gqa_last_error().decode() != ""


def test_fp8_page_bytes(lib):
    """Codes of page_size rows of H_kv*d bytes, then page_size fp32 scales."""
    assert lib.gqa_fp8_page_bytes(16, 8, 128) == 16 * 8 * 128 + 64
    assert lib.gqa_fp8_page_bytes(0, 8, 128) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULLP), (dict(pool=None), NULLP), (dict(tbl=None), NULLP), (dict(x=MIS), ALIGN),
    (dict(pool=ctypes.c_void_p(0x10008)), ALIGN), (dict(sl=ctypes.c_void_p(0x10002)), ALIGN),
    (dict(B=0), SHAPE), (dict(d=12), UNSUP), (dict(page=0), SHAPE), (dict(max_blocks=1), SHAPE),
])
def test_kv_quantize_fp8_rejects_before_launch(lib, kw, code):
    a = dict(x=A, sl=None, tbl=A, pool=A, B=2, S_max=64, H_kv=8, d=128, page=16, num_pages=8,
             max_blocks=4)
    a.update(kw)
    assert lib.gqa_kv_quantize_fp8(a["x"], a["sl"], a["tbl"], a["pool"], a["B"], a["S_max"],
                                   a["H_kv"], a["d"], a["page"], a["num_pages"],
                                   a["max_blocks"], None) == code
    assert lib.gqa_last_error().decode() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULLP), (dict(pool=None), NULLP), (dict(tbl=None), NULLP), (dict(x=MIS), ALIGN),
    (dict(pool=ctypes.c_void_p(0x10008)), ALIGN), (dict(sl=ctypes.c_void_p(0x10002)), ALIGN),
    (dict(B=0), SHAPE), (dict(d=12), UNSUP), (dict(page=0), SHAPE), (dict(max_blocks=1), SHAPE),
])
def test_kv_dequantize_fp8_rejects_before_launch(lib, kw, code):
    a = dict(x=A, sl=None, tbl=A, pool=A, B=2, S_max=64, H_kv=8, d=128, page=16, num_pages=8,
             max_blocks=4)
    a.update(kw)
    assert lib.gqa_kv_dequantize_fp8(a["pool"], a["sl"], a["tbl"], a["x"], a["B"], a["S_max"],
                                     a["H_kv"], a["d"], a["page"], a["num_pages"],
                                     a["max_blocks"], None) == code
    assert lib.gqa_last_error().decode() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(d=32), UNSUP), (dict(page=24), SHAPE), (dict(tbl=None), NULLP), (dict(q=MIS), ALIGN),
    (dict(ws=None), WS), (dict(H_kv=3), SHAPE),
])
def test_decode_paged_fp8_rejects_before_launch(lib, kw, code):
    a = dict(q=A, k=A, v=A, tbl=A, sl=None, o=A, lse=A, B=1, T=1, H_q=8, H_kv=2, d=128, page=16,
             num_pages=8, max_blocks=4, scale=0.088, splits=0, ws=A, ws_bytes=1 << 30)
    a.update(kw)
    assert lib.gqa_attn_decode_paged_fp8(a["q"], a["k"], a["v"], a["tbl"], a["sl"], a["o"],
                                         a["lse"], a["B"], a["T"], a["H_q"], a["H_kv"], a["d"],
                                         a["page"], a["num_pages"], a["max_blocks"], a["scale"],
                                         a["splits"], a["ws"], a["ws_bytes"], None) == code


def test_binding_raises_with_detail():
    with pytest.raises(g.GQAError) as ei:
        g.decode_plan(1, 64, 7, 128, 1024, 0)
    assert ei.value.name == "GQA_ERR_BAD_SHAPE" and "divide" in ei.value.detail


def test_stream_read_rejects_before_launch(lib):
    """The streaming-read calibration checks its buffer, sink and size on the host."""
    assert lib.gqa_stream_read(None, 1024, A, None) == NULLP
    assert lib.gqa_stream_read(A, 1024, None, None) == NULLP
    assert lib.gqa_stream_read(ctypes.c_void_p(0x10008), 1024, A, None) == ALIGN
    assert lib.gqa_stream_read(A, 1024, ctypes.c_void_p(0x10002), None) == ALIGN
    assert lib.gqa_stream_read(A, 0, A, None) == SHAPE
    assert lib.gqa_stream_read(A, 1000, A, None) == SHAPE      # not a multiple of 16
    sink = lib.gqa_stream_read_sink_bytes()
    assert sink > 0 and sink % 4 == 0


def test_mfma_rate_rejects_before_launch(lib):
    """The matrix-core calibration checks its operands, sink, size and round count on the
    host, and leaves the FLOP count untouched when it refuses."""
    flop = ctypes.c_double(-1.0)
    fp = ctypes.byref(flop)
    assert lib.gqa_mfma_rate(None, 1024, 4, A, fp, None) == NULLP
    assert lib.gqa_mfma_rate(A, 1024, 4, None, fp, None) == NULLP
    assert lib.gqa_mfma_rate(ctypes.c_void_p(0x10008), 1024, 4, A, fp, None) == ALIGN
    assert lib.gqa_mfma_rate(A, 1024, 4, ctypes.c_void_p(0x10002), fp, None) == ALIGN
    assert lib.gqa_mfma_rate(A, 240, 4, A, fp, None) == SHAPE        # under 256 bytes
    assert lib.gqa_mfma_rate(A, 1000, 4, A, fp, None) == SHAPE       # not a multiple of 16
    assert lib.gqa_mfma_rate(A, 1024, 0, A, fp, None) == SHAPE
    assert lib.gqa_mfma_rate(A, 1024, (1 << 20) + 1, A, fp, None) == SHAPE
    assert flop.value == -1.0
    sink = lib.gqa_mfma_rate_sink_bytes()
    # one float per thread of 256 workgroups of 512 threads
    assert sink == 256 * 512 * 4


def _noalloc(lib, q=A, k=A, v=A, seqlens=None, o=A, lse=A, B=1, H_q=64, H_kv=8, d=128, S=64,
             scale=0.088, splits=32):
    return lib.gqa_attn_decode_noalloc(q, k, v, seqlens, o, lse, B, H_q, H_kv, d, S, scale,
                                       splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULLP), (dict(o=None), NULLP), (dict(lse=None), NULLP),
    (dict(q=MIS), ALIGN), (dict(H_kv=3), SHAPE), (dict(d=16), UNSUP), (dict(splits=-1), SPLITS),
    (dict(scale=float("nan")), SCALE),
    # the most partitions the plan allows: 65535 + B - 1 slots x 64 heads x (256 + 8) bytes of
    # states, beyond the library's own 16 MiB
    (dict(splits=65535), WS),
])
def test_noalloc_decode_rejects_before_launch(lib, kw, code):
    """The no-allocation decode validates like gqa_attn_decode and refuses a plan whose
    workspace exceeds its own array, all before touching the GPU."""
    assert _noalloc(lib, **kw) == code
    assert lib.gqa_last_error().decode() != ""


def test_noalloc_limit_holds_the_llama_decodes(lib):
    """The 16 MiB array holds the workspace of the Llama decode and of the B = 8 batch."""
    limit = lib.gqa_decode_noalloc_max_workspace()
    assert limit == 16 << 20
    for B, S, splits in ((1, 32768, 32), (8, 92610, 64)):
        plan = g.decode_plan(B, 64, 8, 128, S, splits)
        assert plan["workspace_bytes"] <= limit, (B, S, plan)
