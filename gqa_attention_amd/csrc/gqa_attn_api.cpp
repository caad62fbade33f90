// gqa_attn_api.cpp -- the C ABI of libgqa_attn.so: argument checks, split-KV
// planning, workspace layout and kernel launches.  Every check runs on the
// host before the first launch, so a call with bad arguments returns an error
// code without touching the GPU.  Nothing here allocates or synchronises.
#include "../../include/gqa_attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "gqa_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_err[0] = '\0';
    return GQA_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

constexpr int kMaxSplits = 65535;
constexpr int kGridYZ = 65535;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kPagedTile = 16;         // a page holds whole 16-key tiles of the decode sweep
constexpr int kMaxPage = 1 << 16;

bool decode_head_size_ok(int d) { return d == 32 || d == 64 || d == 128; }

struct Plan {
    int units;          // partitions of the batch's tiles (workgroups per head-group row)
    int hpw;            // KV heads swept together by one workgroup
    int cb;             // 16-column blocks per wave (2 when a KV head has > 16 rows)
    int slots;          // partial-state slots per query head: units + B - 1
    size_t off_m2, off_l, off_o, bytes;
};

constexpr int kDecodeWaves = 8;        // waves per decode workgroup
constexpr int kDecodeTile = 16;        // keys per tile of the decode sweep
constexpr int kTargetWorkgroups = 256; // auto partition count: one workgroup per MI355X CU
constexpr int kMaxDecodeTokens = 16;   // query tokens per sequence of a multi-token decode

int check_heads(int B, int H_q, int H_kv) {
    if (B <= 0 || H_q <= 0 || H_kv <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "B=%d, H_q=%d, H_kv=%d must all be positive", B, H_q, H_kv);
    if (H_q % H_kv != 0)
        return fail(GQA_ERR_BAD_SHAPE, "H_kv=%d does not divide H_q=%d", H_kv, H_q);
    return GQA_OK;
}

int make_plan(int B, int T, int H_q, int H_kv, int d, int S_max, int num_splits, Plan *pl) {
    int rc = check_heads(B, H_q, H_kv);
    if (rc) return rc;
    if (T < 1 || T > kMaxDecodeTokens)
        return fail(GQA_ERR_BAD_SHAPE, "T_q=%d outside [1, %d]", T, kMaxDecodeTokens);
    if (!decode_head_size_ok(d))
        return fail(GQA_ERR_UNSUPPORTED, "decode head size d=%d (supported: 32, 64, 128)", d);
    if (S_max <= 0) return fail(GQA_ERR_BAD_SHAPE, "S_max=%d must be positive", S_max);
    if (B > gqa::kMaxDecodeBatch)
        return fail(GQA_ERR_BAD_SHAPE, "decode batch B=%d exceeds %d", B, gqa::kMaxDecodeBatch);
    const long tiles = (long)B * ((S_max + kDecodeTile - 1) / kDecodeTile);
    if (tiles > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B * ceil(S_max/16) = %ld exceeds 2^31 - 1", tiles);
    if (num_splits < 0 || num_splits > kMaxSplits)
        return fail(GQA_ERR_SPLITS, "num_splits=%d outside [0, %d]", num_splits, kMaxSplits);
    const int G = H_q / H_kv;
    // a wave folds up to 2 blocks of 16 of a KV head's G * T rows; more run as further
    // workgroup rows
    const int cb = (long)G * T > 16 ? 2 : 1;
    const long n_hg = ((long)G * T + 16 * cb - 1) / (16 * cb);
    // KV heads per workgroup: the largest power of two <= 8 that divides H_kv; the
    // workgroup's 8 waves are spread evenly over them
    int hpw = kDecodeWaves;
    while (H_kv % hpw) hpw /= 2;
    const long rows = (long)(H_kv / hpw) * n_hg;
    if (rows > kGridYZ)
        return fail(GQA_ERR_BAD_SHAPE, "H_kv/%d * ceil(G/16) = %ld exceeds %d", hpw, rows, kGridYZ);
    // at least num_splits partitions, and at least enough workgroups to fill the device
    const long fill = (kTargetWorkgroups + rows - 1) / rows;
    const long units = num_splits > fill ? num_splits : fill;
    pl->units = (int)units;
    pl->hpw = hpw;
    pl->cb = cb;
    pl->slots = (int)(units + B - 1);
    const size_t states = (size_t)pl->slots * H_q * T;
    pl->off_m2 = align256((size_t)B * 2 * sizeof(int32_t));
    pl->off_l = pl->off_m2 + align256(states * sizeof(float));
    pl->off_o = pl->off_l + align256(states * sizeof(float));
    pl->bytes = pl->off_o + align256(states * (size_t)d * sizeof(uint16_t));   // O in bf16
    return GQA_OK;
}

int check_scale(float scale) {
    if (!std::isfinite(scale) || scale < 0.f)
        return fail(GQA_ERR_SCALE, "softmax_scale=%g must be finite and >= 0", (double)scale);
    return GQA_OK;
}

int check_workspace(const void *ws, size_t bytes, const Plan &pl) {
    if (!ws) return fail(GQA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.bytes);
    if (!aligned(ws, 256)) return fail(GQA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (bytes < pl.bytes)
        return fail(GQA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, pl.bytes);
    return GQA_OK;
}

int check_bf16(const void *p, const char *name) {
    if (!p) return fail(GQA_ERR_NULL_POINTER, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(GQA_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
    return GQA_OK;
}

int check_f32(const void *p, const char *name) {
    if (!p) return fail(GQA_ERR_NULL_POINTER, "%s is NULL", name);
    if (!aligned(p, 4)) return fail(GQA_ERR_ALIGNMENT, "%s is not 4-byte aligned", name);
    return GQA_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(GQA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return GQA_OK;
}

int decode_common_checks(const void *q, const void *k, const void *v, const int32_t *seqlens,
                         float scale) {
    int rc;
    if ((rc = check_bf16(q, "q")) || (rc = check_bf16(k, "k_cache")) ||
        (rc = check_bf16(v, "v_cache")))
        return rc;
    if (seqlens && !aligned(seqlens, 4)) return fail(GQA_ERR_ALIGNMENT, "seqlens misaligned");
    return check_scale(scale);
}

gqa::DecodeSplitArgs split_args(const void *q, const void *k, const void *v,
                                const int32_t *seqlens, int B, int H_q, int H_kv, int d, int S_max,
                                float scale, const Plan &pl, void *ws, int T = 1) {
    char *base = static_cast<char *>(ws);
    gqa::DecodeSplitArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.seqlens = seqlens;
    a.seg = reinterpret_cast<int32_t *>(base);
    a.part_m2 = reinterpret_cast<float *>(base + pl.off_m2);
    a.part_l = reinterpret_cast<float *>(base + pl.off_l);
    a.part_o = reinterpret_cast<uint16_t *>(base + pl.off_o);
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.d = d;
    a.S_max = S_max;
    a.T = T;
    a.units = pl.units;
    a.hpw = pl.hpw;
    a.cb = pl.cb;
    a.scale_log2 = scale * kLog2e;
    a.block_table = nullptr;
    a.page = 0;
    a.num_pages = 0;
    a.max_blocks = 0;
    a.fp8 = 0;
    a.page_bytes = 0;
    return a;
}

// uniform_tiles: the 16-key tiles of every sequence when all have the same length (seqlens
// NULL: S_max), which lets the merge find each sequence's states from the plan alone; 0
// when the lengths live on the device (the merge then reads the split kernel's slot table).
gqa::MergeArgs combine_args(void *o, float *lse, int B, int H_q, int d, const Plan &pl,
                            const void *ws, int T = 1, int uniform_tiles = 0) {
    const char *base = static_cast<const char *>(ws);
    gqa::MergeArgs m;
    m.part_m2 = reinterpret_cast<const float *>(base + pl.off_m2);
    m.part_l = reinterpret_cast<const float *>(base + pl.off_l);
    m.part_o = base + pl.off_o;
    m.o_bf16 = 1;
    m.uniform_tiles = uniform_tiles;
    m.units = pl.units;
    m.seg = reinterpret_cast<const int32_t *>(base);
    m.counts = nullptr;
    m.P = pl.slots;
    m.batch_stride = 0;
    m.head_stride = 1;                  // workspace: [slot][H_q * T]
    m.state_stride = (long)H_q * T;
    m.o = static_cast<uint16_t *>(o);
    m.lse = lse;
    m.B = B;
    m.H_q = H_q;
    m.d = d;
    m.T = T;
    return m;
}

// Tiles of every sequence when seqlens is NULL (all of length S_max), else 0.
int uniform_tiles(const int32_t *seqlens, int S_max) {
    return seqlens ? 0 : (S_max + kDecodeTile - 1) / kDecodeTile;
}

// A paged cache for prefill (block_table null: contiguous).
struct PagedCache {
    const int32_t *block_table = nullptr;
    int page = 0, num_pages = 0, max_blocks = 0;
    const int32_t *q_starts = nullptr;
    int q_start_max = 0;
};

// Causal prefill of T query rows (tokens q_start .. q_start + T - 1) against a cache of
// S rows per sequence; the callers have checked T > 0, S > 0 and 0 <= q_start <= S - T
// (and, for a paged cache, its pool and table).
int prefill(const void *q, const void *k, const void *v, void *o, float *lse, int B, int T,
            int q_start, int S, int H_q, int H_kv, int d, float softmax_scale, void *stream,
            const PagedCache &pc = PagedCache()) {
    int rc;
    if ((rc = check_heads(B, H_q, H_kv))) return rc;
    if (d != 128) return fail(GQA_ERR_UNSUPPORTED, "prefill head size d=%d (supported: 128)", d);
    const long n_qb = (T + 127) / 128;
    if (n_qb * (long)B * H_q > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B*H_q*ceil(T_q/128) exceeds the grid limit");
    if ((rc = check_bf16(q, "q")) || (rc = check_bf16(k, "k")) || (rc = check_bf16(v, "v")) ||
        (rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse")))
        return rc;
    if ((rc = check_scale(softmax_scale))) return rc;
    gqa::PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = B;
    a.S = S;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.d = d;
    a.T = T;
    a.q_start = q_start;
    a.scale_log2 = softmax_scale * kLog2e;
    a.block_table = pc.block_table;
    a.page = pc.page;
    a.num_pages = pc.num_pages;
    a.max_blocks = pc.max_blocks;
    a.q_starts = pc.q_starts;
    a.q_start_max = pc.q_start_max;
    if ((rc = hip_status(gqa::launch_prefill_causal(a, static_cast<hipStream_t>(stream)),
                         "prefill_causal")))
        return rc;
    return ok();
}

// Paged decode over bf16 pools (fp8 = 0) or FP8 pages (fp8 = 1).
int decode_paged(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                 const int32_t *seqlens, void *o, float *lse, int B, int T_q, int H_q, int H_kv,
                 int d, int page_size, int num_pages, int max_blocks, float softmax_scale,
                 int num_splits, void *workspace, size_t workspace_bytes, void *stream, int fp8) {
    if (page_size < kPagedTile || page_size % kPagedTile != 0 || page_size > kMaxPage)
        return fail(GQA_ERR_BAD_SHAPE, "page_size=%d must be a multiple of %d in [%d, %d]",
                    page_size, kPagedTile, kPagedTile, kMaxPage);
    if (num_pages <= 0 || max_blocks <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "num_pages=%d and max_blocks=%d must be positive",
                    num_pages, max_blocks);
    if ((long)num_pages * page_size > 0x7FFFFFFFL || (long)max_blocks * page_size > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE,
                    "num_pages*page_size and max_blocks*page_size must fit in 31 bits");
    if (fp8 && d != 64 && d != 128)
        return fail(GQA_ERR_UNSUPPORTED, "FP8 decode head size d=%d (supported: 64, 128)", d);
    const int S_max = max_blocks * page_size;
    Plan pl;
    int rc;
    if ((rc = make_plan(B, T_q, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = decode_common_checks(q, k_pool, v_pool, seqlens, softmax_scale))) return rc;
    if (!block_table) return fail(GQA_ERR_NULL_POINTER, "block_table is NULL");
    if (!aligned(block_table, 4)) return fail(GQA_ERR_ALIGNMENT, "block_table misaligned");
    if ((rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse"))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, pl))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto a = split_args(q, k_pool, v_pool, seqlens, B, H_q, H_kv, d, S_max, softmax_scale, pl,
                        workspace, T_q);
    a.block_table = block_table;
    a.page = page_size;
    a.num_pages = num_pages;
    a.max_blocks = max_blocks;
    a.fp8 = fp8;
    a.page_bytes = fp8 ? (size_t)page_size * H_kv * d + 4u * (size_t)page_size : 0;
    if ((rc = hip_status(gqa::launch_decode_split(a, s), "decode_split (paged)"))) return rc;
    auto m = combine_args(o, lse, B, H_q, d, pl, workspace, T_q, uniform_tiles(seqlens, S_max));
    if ((rc = hip_status(gqa::launch_lse_merge(m, s), "lse_merge"))) return rc;
    return ok();
}

}  // namespace

extern "C" {

const char *gqa_status_string(int status) {
    switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL_POINTER: return "GQA_ERR_NULL_POINTER";
    case GQA_ERR_BAD_SHAPE: return "GQA_ERR_BAD_SHAPE";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_SPLITS: return "GQA_ERR_SPLITS";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
    case GQA_ERR_ALIGNMENT: return "GQA_ERR_ALIGNMENT";
    case GQA_ERR_SCALE: return "GQA_ERR_SCALE";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
    default: return "GQA_ERR_UNKNOWN";
    }
}

const char *gqa_last_error(void) { return g_err; }

const char *gqa_version(void) { return "gqa_attn 0.2.0 (gfx950)"; }

int gqa_device_info(int device, int *compute_units, int *clock_khz, char *arch, size_t arch_len) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
    if (device < 0 || device >= n)
        return fail(GQA_ERR_BAD_SHAPE, "device %d outside [0, %d)", device, n);
    if (compute_units &&
        (e = hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount,
                                   device)) != hipSuccess)
        return fail(GQA_ERR_HIP, "compute-unit count: %s", hipGetErrorString(e));
    if (clock_khz &&
        (e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, device)) != hipSuccess)
        return fail(GQA_ERR_HIP, "clock rate: %s", hipGetErrorString(e));
    if (arch && arch_len > 0) {
        hipDeviceProp_t prop;
        if ((e = hipGetDeviceProperties(&prop, device)) != hipSuccess)
            return fail(GQA_ERR_HIP, "device properties: %s", hipGetErrorString(e));
        std::snprintf(arch, arch_len, "%s", prop.gcnArchName);
    }
    return ok();
}

size_t gqa_stream_read_sink_bytes(void) { return (size_t)gqa::hbm_read_blocks() * sizeof(uint32_t); }

int gqa_stream_read(const void *buf, size_t bytes, void *sink, void *stream) {
    if (!buf) return fail(GQA_ERR_NULL_POINTER, "buf is NULL");
    if (!sink) return fail(GQA_ERR_NULL_POINTER, "sink is NULL");
    if (!aligned(buf, 16)) return fail(GQA_ERR_ALIGNMENT, "buf is not 16-byte aligned");
    if (!aligned(sink, 4)) return fail(GQA_ERR_ALIGNMENT, "sink is not 4-byte aligned");
    if (bytes == 0 || bytes % 16 != 0)
        return fail(GQA_ERR_BAD_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    int rc;
    if ((rc = hip_status(gqa::launch_hbm_read(buf, bytes, static_cast<uint32_t *>(sink),
                                              static_cast<hipStream_t>(stream)),
                         "hbm_read")))
        return rc;
    return ok();
}

size_t gqa_mfma_rate_sink_bytes(void) { return (size_t)gqa::mfma_rate_threads() * sizeof(float); }

int gqa_mfma_rate(const void *ops, size_t bytes, int iters, void *sink, double *flop_out,
                  void *stream) {
    if (!ops) return fail(GQA_ERR_NULL_POINTER, "ops is NULL");
    if (!sink) return fail(GQA_ERR_NULL_POINTER, "sink is NULL");
    if (!aligned(ops, 16)) return fail(GQA_ERR_ALIGNMENT, "ops is not 16-byte aligned");
    if (!aligned(sink, 4)) return fail(GQA_ERR_ALIGNMENT, "sink is not 4-byte aligned");
    if (bytes < 256 || bytes % 16 != 0)
        return fail(GQA_ERR_BAD_SHAPE, "bytes=%zu must be a multiple of 16 and at least 256", bytes);
    if (iters < 1 || iters > (1 << 20))
        return fail(GQA_ERR_BAD_SHAPE, "iters=%d outside [1, 1048576]", iters);
    int rc;
    if ((rc = hip_status(gqa::launch_mfma_rate(ops, bytes, iters, static_cast<float *>(sink),
                                               static_cast<hipStream_t>(stream)),
                         "mfma_rate")))
        return rc;
    if (flop_out) *flop_out = gqa::mfma_rate_flop(iters);
    return ok();
}

int gqa_decode_plan(int B, int H_q, int H_kv, int d, int S_max, int num_splits,
                    int *partitions_out, int *states_out, size_t *workspace_bytes_out) {
    Plan pl;
    int rc = make_plan(B, 1, H_q, H_kv, d, S_max, num_splits, &pl);
    if (rc) return rc;
    if (partitions_out) *partitions_out = pl.units;
    if (states_out) *states_out = pl.slots;
    if (workspace_bytes_out) *workspace_bytes_out = pl.bytes;
    return ok();
}

int gqa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seqlens, int B, int H_q, int H_kv, int d, int S_max,
                        float softmax_scale, int num_splits, void *workspace,
                        size_t workspace_bytes, void *stream) {
    Plan pl;
    int rc;
    if ((rc = make_plan(B, 1, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = decode_common_checks(q, k_cache, v_cache, seqlens, softmax_scale))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, pl))) return rc;
    auto a = split_args(q, k_cache, v_cache, seqlens, B, H_q, H_kv, d, S_max, softmax_scale, pl,
                        workspace);
    if ((rc = hip_status(gqa::launch_decode_split(a, static_cast<hipStream_t>(stream)),
                         "decode_split")))
        return rc;
    return ok();
}

int gqa_decode_combine(void *o, float *lse, int B, int H_q, int H_kv, int d, int S_max,
                       int num_splits, const void *workspace, size_t workspace_bytes,
                       void *stream) {
    Plan pl;
    int rc;
    if ((rc = make_plan(B, 1, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse"))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, pl))) return rc;
    auto m = combine_args(o, lse, B, H_q, d, pl, workspace);
    if ((rc = hip_status(gqa::launch_lse_merge(m, static_cast<hipStream_t>(stream)), "lse_merge")))
        return rc;
    return ok();
}

int gqa_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *seqlens, void *o, float *lse, int B, int H_q, int H_kv, int d,
                    int S_max, float softmax_scale, int num_splits, void *workspace,
                    size_t workspace_bytes, void *stream) {
    Plan pl;
    int rc;
    if ((rc = make_plan(B, 1, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = decode_common_checks(q, k_cache, v_cache, seqlens, softmax_scale))) return rc;
    if ((rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse"))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, pl))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto a = split_args(q, k_cache, v_cache, seqlens, B, H_q, H_kv, d, S_max, softmax_scale, pl,
                        workspace);
    if ((rc = hip_status(gqa::launch_decode_split(a, s), "decode_split"))) return rc;
    auto m = combine_args(o, lse, B, H_q, d, pl, workspace, 1, uniform_tiles(seqlens, S_max));
    if ((rc = hip_status(gqa::launch_lse_merge(m, s), "lse_merge"))) return rc;
    return ok();
}

int gqa_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seqlens, void *o, float *lse, int B, int H_q, int H_kv,
                            int d, int S_max, float softmax_scale, int num_splits, void *stream) {
    Plan pl;
    int rc;
    if ((rc = make_plan(B, 1, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = decode_common_checks(q, k_cache, v_cache, seqlens, softmax_scale))) return rc;
    if ((rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse"))) return rc;
    if (pl.bytes > gqa::noalloc_scratch_bytes())
        return fail(GQA_ERR_WORKSPACE,
                    "this decode needs %zu bytes of workspace; the library's own holds %zu "
                    "(use gqa_attn_decode with a caller workspace)",
                    pl.bytes, gqa::noalloc_scratch_bytes());
    void *ws = nullptr;
    hipError_t e = gqa::noalloc_scratch(&ws);
    if (e != hipSuccess)
        return fail(GQA_ERR_HIP, "device workspace lookup failed: %s", hipGetErrorString(e));
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto a = split_args(q, k_cache, v_cache, seqlens, B, H_q, H_kv, d, S_max, softmax_scale, pl,
                        ws);
    if ((rc = hip_status(gqa::launch_decode_split(a, s), "decode_split"))) return rc;
    auto m = combine_args(o, lse, B, H_q, d, pl, ws, 1, uniform_tiles(seqlens, S_max));
    if ((rc = hip_status(gqa::launch_lse_merge(m, s), "lse_merge"))) return rc;
    return ok();
}

size_t gqa_decode_noalloc_max_workspace(void) { return gqa::noalloc_scratch_bytes(); }

int gqa_attn_decode_paged(const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_table, const int32_t *seqlens, void *o, float *lse,
                          int B, int T_q, int H_q, int H_kv, int d, int page_size, int num_pages,
                          int max_blocks, float softmax_scale, int num_splits, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return decode_paged(q, k_pool, v_pool, block_table, seqlens, o, lse, B, T_q, H_q, H_kv, d,
                        page_size, num_pages, max_blocks, softmax_scale, num_splits, workspace,
                        workspace_bytes, stream, 0);
}

size_t gqa_fp8_page_bytes(int page_size, int H_kv, int d) {
    if (page_size <= 0 || H_kv <= 0 || d <= 0) return 0;
    return (size_t)page_size * H_kv * d + 4u * (size_t)page_size;
}

int gqa_attn_decode_paged_fp8(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *block_table, const int32_t *seqlens, void *o,
                              float *lse, int B, int T_q, int H_q, int H_kv, int d, int page_size,
                              int num_pages, int max_blocks, float softmax_scale, int num_splits,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return decode_paged(q, k_pool, v_pool, block_table, seqlens, o, lse, B, T_q, H_q, H_kv, d,
                        page_size, num_pages, max_blocks, softmax_scale, num_splits, workspace,
                        workspace_bytes, stream, 1);
}

int gqa_kv_quantize_fp8(const void *x, const int32_t *seqlens, const int32_t *block_table,
                        void *pool, int B, int S_max, int H_kv, int d, int page_size,
                        int num_pages, int max_blocks, void *stream) {
    if (B <= 0 || S_max <= 0 || H_kv <= 0 || d <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "B=%d, S_max=%d, H_kv=%d, d=%d must be positive", B, S_max,
                    H_kv, d);
    if (d % 8 != 0) return fail(GQA_ERR_UNSUPPORTED, "FP8 quantisation needs d %% 8 == 0 (d=%d)", d);
    if (page_size <= 0 || num_pages <= 0 || max_blocks <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "page_size=%d, num_pages=%d, max_blocks=%d must be positive",
                    page_size, num_pages, max_blocks);
    if ((long)max_blocks * page_size < S_max)
        return fail(GQA_ERR_BAD_SHAPE, "max_blocks*page_size=%ld is below S_max=%d",
                    (long)max_blocks * page_size, S_max);
    if ((long)B * S_max > 0x7FFFFFFFL || (long)H_kv * d > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B*S_max and H_kv*d must fit in 31 bits");
    int rc;
    if ((rc = check_bf16(x, "x"))) return rc;
    if (!pool) return fail(GQA_ERR_NULL_POINTER, "pool is NULL");
    if (!aligned(pool, 16)) return fail(GQA_ERR_ALIGNMENT, "pool is not 16-byte aligned");
    if (!block_table) return fail(GQA_ERR_NULL_POINTER, "block_table is NULL");
    if (!aligned(block_table, 4)) return fail(GQA_ERR_ALIGNMENT, "block_table misaligned");
    if (seqlens && !aligned(seqlens, 4)) return fail(GQA_ERR_ALIGNMENT, "seqlens misaligned");
    gqa::KvQuantArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.seqlens = seqlens;
    a.block_table = block_table;
    a.pool = static_cast<uint8_t *>(pool);
    a.B = B;
    a.S_max = S_max;
    a.H_kv = H_kv;
    a.d = d;
    a.page = page_size;
    a.num_pages = num_pages;
    a.max_blocks = max_blocks;
    a.page_bytes = gqa_fp8_page_bytes(page_size, H_kv, d);
    if ((rc = hip_status(gqa::launch_kv_quantize_fp8(a, static_cast<hipStream_t>(stream)),
                         "kv_quantize_fp8")))
        return rc;
    return ok();
}

int gqa_kv_dequantize_fp8(const void *pool, const int32_t *seqlens, const int32_t *block_table,
                          void *x, int B, int S_max, int H_kv, int d, int page_size, int num_pages,
                          int max_blocks, void *stream) {
    if (B <= 0 || S_max <= 0 || H_kv <= 0 || d <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "B=%d, S_max=%d, H_kv=%d, d=%d must be positive", B, S_max,
                    H_kv, d);
    if (d % 8 != 0) return fail(GQA_ERR_UNSUPPORTED, "FP8 dequantisation needs d %% 8 == 0 (d=%d)", d);
    if (page_size <= 0 || num_pages <= 0 || max_blocks <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "page_size=%d, num_pages=%d, max_blocks=%d must be positive",
                    page_size, num_pages, max_blocks);
    if ((long)max_blocks * page_size < S_max)
        return fail(GQA_ERR_BAD_SHAPE, "max_blocks*page_size=%ld is below S_max=%d",
                    (long)max_blocks * page_size, S_max);
    if ((long)B * S_max > 0x7FFFFFFFL || (long)H_kv * d > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B*S_max and H_kv*d must fit in 31 bits");
    int rc;
    if ((rc = check_bf16(x, "x"))) return rc;
    if (!pool) return fail(GQA_ERR_NULL_POINTER, "pool is NULL");
    if (!aligned(pool, 16)) return fail(GQA_ERR_ALIGNMENT, "pool is not 16-byte aligned");
    if (!block_table) return fail(GQA_ERR_NULL_POINTER, "block_table is NULL");
    if (!aligned(block_table, 4)) return fail(GQA_ERR_ALIGNMENT, "block_table misaligned");
    if (seqlens && !aligned(seqlens, 4)) return fail(GQA_ERR_ALIGNMENT, "seqlens misaligned");
    gqa::KvDequantArgs a;
    a.pool = static_cast<const uint8_t *>(pool);
    a.seqlens = seqlens;
    a.block_table = block_table;
    a.x = static_cast<uint16_t *>(x);
    a.B = B;
    a.S_max = S_max;
    a.H_kv = H_kv;
    a.d = d;
    a.page = page_size;
    a.num_pages = num_pages;
    a.max_blocks = max_blocks;
    a.page_bytes = gqa_fp8_page_bytes(page_size, H_kv, d);
    if ((rc = hip_status(gqa::launch_kv_dequantize_fp8(a, static_cast<hipStream_t>(stream)),
                         "kv_dequantize_fp8")))
        return rc;
    return ok();
}

int gqa_decode_tokens_plan(int B, int T_q, int H_q, int H_kv, int d, int S_max, int num_splits,
                           int *partitions_out, int *states_out, size_t *workspace_bytes_out) {
    Plan pl;
    int rc = make_plan(B, T_q, H_q, H_kv, d, S_max, num_splits, &pl);
    if (rc) return rc;
    if (partitions_out) *partitions_out = pl.units;
    if (states_out) *states_out = pl.slots;
    if (workspace_bytes_out) *workspace_bytes_out = pl.bytes;
    return ok();
}

int gqa_attn_decode_tokens(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seqlens, void *o, float *lse, int B, int T_q, int H_q,
                           int H_kv, int d, int S_max, float softmax_scale, int num_splits,
                           void *workspace, size_t workspace_bytes, void *stream) {
    Plan pl;
    int rc;
    if ((rc = make_plan(B, T_q, H_q, H_kv, d, S_max, num_splits, &pl))) return rc;
    if ((rc = decode_common_checks(q, k_cache, v_cache, seqlens, softmax_scale))) return rc;
    if ((rc = check_bf16(o, "o")) || (rc = check_f32(lse, "lse"))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, pl))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto a = split_args(q, k_cache, v_cache, seqlens, B, H_q, H_kv, d, S_max, softmax_scale, pl,
                        workspace, T_q);
    if ((rc = hip_status(gqa::launch_decode_split(a, s), "decode_split (tokens)"))) return rc;
    auto m = combine_args(o, lse, B, H_q, d, pl, workspace, T_q, uniform_tiles(seqlens, S_max));
    if ((rc = hip_status(gqa::launch_lse_merge(m, s), "lse_merge"))) return rc;
    return ok();
}

int gqa_lse_merge(const float *part_m2, const float *part_l, const float *part_o,
                  const int32_t *split_counts, int max_splits, void *o, float *lse, int B, int H_q,
                  int d, void *stream) {
    int rc;
    if (B <= 0 || H_q <= 0) return fail(GQA_ERR_BAD_SHAPE, "B=%d, H_q=%d must be positive", B, H_q);
    if (B > kGridYZ) return fail(GQA_ERR_BAD_SHAPE, "B=%d exceeds %d", B, kGridYZ);
    if (!decode_head_size_ok(d))
        return fail(GQA_ERR_UNSUPPORTED, "merge head size d=%d (supported: 32, 64, 128)", d);
    if (max_splits <= 0 || max_splits > kMaxSplits)
        return fail(GQA_ERR_SPLITS, "max_splits=%d outside [1, %d]", max_splits, kMaxSplits);
    if ((rc = check_f32(part_m2, "part_m2")) || (rc = check_f32(part_l, "part_l")) ||
        (rc = check_f32(part_o, "part_o")) || (rc = check_bf16(o, "o")) ||
        (rc = check_f32(lse, "lse")))
        return rc;
    if (!aligned(part_o, 16)) return fail(GQA_ERR_ALIGNMENT, "part_o is not 16-byte aligned");
    if (split_counts && !aligned(split_counts, 4))
        return fail(GQA_ERR_ALIGNMENT, "split_counts misaligned");
    gqa::MergeArgs m;
    m.part_m2 = part_m2;
    m.part_l = part_l;
    m.part_o = part_o;
    m.o_bf16 = 0;
    m.uniform_tiles = 0;
    m.units = 0;
    m.counts = split_counts;
    m.seg = nullptr;
    m.T = 1;
    m.P = max_splits;
    m.batch_stride = (long)H_q * max_splits;   // caller's partials: [B][H_q][P]
    m.head_stride = max_splits;
    m.state_stride = 1;
    m.o = static_cast<uint16_t *>(o);
    m.lse = lse;
    m.B = B;
    m.H_q = H_q;
    m.d = d;
    if ((rc = hip_status(gqa::launch_lse_merge(m, static_cast<hipStream_t>(stream)), "lse_merge")))
        return rc;
    return ok();
}

int gqa_attn_prefill_causal(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int S, int H_q, int H_kv, int d, float softmax_scale,
                            void *stream) {
    if (S <= 0) return fail(GQA_ERR_BAD_SHAPE, "S=%d must be positive", S);
    return prefill(q, k, v, o, lse, B, S, 0, S, H_q, H_kv, d, softmax_scale, stream);
}

int gqa_attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache, void *o,
                           float *lse, int B, int T_q, int q_start, int S_kv, int H_q, int H_kv,
                           int d, float softmax_scale, void *stream) {
    if (T_q <= 0 || S_kv <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "T_q=%d and S_kv=%d must be positive", T_q, S_kv);
    if (q_start < 0 || q_start > S_kv - T_q)
        return fail(GQA_ERR_BAD_SHAPE, "q_start=%d outside [0, S_kv - T_q] = [0, %d]", q_start,
                    S_kv - T_q);
    return prefill(q, k_cache, v_cache, o, lse, B, T_q, q_start, S_kv, H_q, H_kv, d,
                   softmax_scale, stream);
}

int gqa_attn_prefill_chunk_paged(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_table, const int32_t *q_starts, void *o,
                                 float *lse, int B, int T_q, int q_start, int H_q, int H_kv, int d,
                                 int page_size, int num_pages, int max_blocks,
                                 float softmax_scale, void *stream) {
    if (T_q <= 0 || q_start < 0)
        return fail(GQA_ERR_BAD_SHAPE, "T_q=%d must be positive and q_start=%d non-negative", T_q,
                    q_start);
    if (page_size < kPagedTile || page_size % kPagedTile != 0 || page_size > kMaxPage)
        return fail(GQA_ERR_BAD_SHAPE, "page_size=%d must be a multiple of %d in [%d, %d]",
                    page_size, kPagedTile, kPagedTile, kMaxPage);
    if (num_pages <= 0 || max_blocks <= 0)
        return fail(GQA_ERR_BAD_SHAPE, "num_pages=%d and max_blocks=%d must be positive",
                    num_pages, max_blocks);
    if ((long)num_pages * page_size > 0x7FFFFFFFL || (long)max_blocks * page_size > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE,
                    "num_pages*page_size and max_blocks*page_size must fit in 31 bits");
    const long keys = (long)q_start + T_q;        // keys the chunk sees: [0, q_start + T_q)
    const long blocks = (keys + page_size - 1) / page_size;
    if (blocks > max_blocks)
        return fail(GQA_ERR_BAD_SHAPE, "q_start+T_q=%ld keys need %ld blocks, the table has %d",
                    keys, blocks, max_blocks);
    if (blocks > gqa::kPrefillMaxPages)
        return fail(GQA_ERR_UNSUPPORTED, "q_start+T_q=%ld keys span %ld blocks (at most %d: use "
                    "larger pages)", keys, blocks, gqa::kPrefillMaxPages);
    if (!block_table) return fail(GQA_ERR_NULL_POINTER, "block_table is NULL");
    if (!aligned(block_table, 4)) return fail(GQA_ERR_ALIGNMENT, "block_table misaligned");
    if (q_starts && !aligned(q_starts, 4)) return fail(GQA_ERR_ALIGNMENT, "q_starts misaligned");
    PagedCache pc;
    pc.block_table = block_table;
    pc.page = page_size;
    pc.num_pages = num_pages;
    pc.max_blocks = max_blocks;
    pc.q_starts = q_starts;
    // the largest start whose keys still fit the table and the staged table row
    const long cap = (long)(max_blocks < gqa::kPrefillMaxPages ? max_blocks : gqa::kPrefillMaxPages)
                     * page_size;
    pc.q_start_max = (int)(cap - T_q);
    return prefill(q, k_pool, v_pool, o, lse, B, T_q, q_start, (int)keys, H_q, H_kv, d,
                   softmax_scale, stream, pc);
}

size_t gqa_prefill_bwd_workspace_bytes(int B, int S, int H_q, int H_kv, int d) {
    if (B <= 0 || S <= 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 || d != 128) return 0;
    return gqa::prefill_bwd_workspace_bytes(B, S, H_q);
}

int gqa_attn_prefill_causal_bwd(const void *q, const void *k, const void *v, const void *o,
                                const float *lse, const void *d_o, void *dq, void *dk, void *dv,
                                int B, int S, int H_q, int H_kv, int d, float softmax_scale,
                                void *workspace, size_t workspace_bytes, void *stream) {
    int rc;
    if ((rc = check_heads(B, H_q, H_kv))) return rc;
    if (S <= 0) return fail(GQA_ERR_BAD_SHAPE, "S=%d must be positive", S);
    if (d != 128)
        return fail(GQA_ERR_UNSUPPORTED, "prefill backward head size d=%d (supported: 128)", d);
    const long n_qb = (S + 255) / 256;
    if (n_qb * (long)B * H_q > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B*H_q*ceil(S/256) exceeds the grid limit");
    if ((long)B * H_q * ((S + 63) / 64) * 4 > 0x7FFFFFFFL)
        return fail(GQA_ERR_BAD_SHAPE, "B*H_q*S exceeds the grid limit");
    if ((rc = check_bf16(q, "q")) || (rc = check_bf16(k, "k")) || (rc = check_bf16(v, "v")) ||
        (rc = check_bf16(o, "o")) || (rc = check_bf16(d_o, "d_o")) || (rc = check_f32(lse, "lse")) ||
        (rc = check_bf16(dq, "dq")) || (rc = check_bf16(dk, "dk")) || (rc = check_bf16(dv, "dv")))
        return rc;
    if ((rc = check_scale(softmax_scale))) return rc;
    const size_t need = gqa::prefill_bwd_workspace_bytes(B, S, H_q);
    if (!workspace) return fail(GQA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 256)) return fail(GQA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
        return fail(GQA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    gqa::BwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.o = static_cast<const uint16_t *>(o);
    a.dout = static_cast<const uint16_t *>(d_o);
    a.lse = lse;
    a.dq = static_cast<uint16_t *>(dq);
    a.dk = static_cast<uint16_t *>(dk);
    a.dv = static_cast<uint16_t *>(dv);
    a.stats = nullptr;
    a.B = B;
    a.S = S;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.d = d;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    if ((rc = hip_status(gqa::launch_prefill_bwd(a, workspace, static_cast<hipStream_t>(stream)),
                         "prefill_causal_bwd")))
        return rc;
    return ok();
}

}  // extern "C"
