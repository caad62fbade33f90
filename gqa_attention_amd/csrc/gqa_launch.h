// gqa_launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Every launcher trusts its arguments: the C ABI layer validates shapes,
// pointers and sizes before calling any of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// Largest batch of one decode launch: every workgroup keeps the running tile counts of the
// batch's sequences in LDS.
constexpr int kMaxDecodeBatch = 8192;

// Split-KV plan: the 16-key tiles of all sequences of the batch, in order, are cut into
// `units` equal contiguous partitions, one workgroup each (per group of `hpw` KV heads and
// 16-row slice of a group's rows, blockIdx.y).  A KV head's rows are its G query heads times
// the T query tokens of a sequence (T = 1: one-token decode), row (h, i) = h * T + i; token
// i is the sequence's position len - T + i and sees keys up to it.  Partition x writes its
// partial state of sequence b (m2, l, O of every row of its KV heads) in state slot x + b;
// states are stored slot-major, [slot][H_q * T] (O: [..][d]), and seg[b] = {first slot,
// count} of b.  A state's O is stored in bf16 (its m2 and l in fp32).
struct DecodeSplitArgs {
    const uint16_t *q, *k, *v;  // bf16 bit patterns; q [B][T][H_q][d]
    const int32_t *seqlens;     // [B] or nullptr
    float *part_m2, *part_l;
    uint16_t *part_o;           // bf16 bits
    int32_t *seg;               // [B][2], written by workgroup (0, 0)
    int B, H_q, H_kv, d, S_max;
    int T;                      // query tokens per sequence
    int units;                  // partitions (workgroups along x)
    int hpw;                    // KV heads per workgroup (divides H_kv and the wave count)
    int cb;                     // 16-column blocks per wave: 2 when G * T > 16, else 1
    float scale_log2;           // softmax_scale * log2(e)
    // Paged cache when block_table is not null: k and v are pools [num_pages][page][H_kv][d]
    // and key t of sequence b is row t % page of page block_table[b * max_blocks + t / page]
    // (page a multiple of 16; S_max = max_blocks * page).
    const int32_t *block_table;
    int page, num_pages, max_blocks;
    // FP8 pages (paged only, d = 64 or 128): k and v are byte pools of pages of page_bytes bytes,
    // [page][H_kv][d] E4M3 codes followed by `page` fp32 per-token scales.
    int fp8;
    size_t page_bytes;
};

// Per-token E4M3 quantisation of a cache x [B][S_max][H_kv][d] (bf16) into the pages of an
// FP8 pool: token t < len(b) of sequence b goes to row t % page of page
// block_table[b][t / page] (an entry outside [0, num_pages) is skipped).
struct KvQuantArgs {
    const uint16_t *x;
    const int32_t *seqlens;     // [B] or nullptr (= S_max)
    const int32_t *block_table; // [B][max_blocks]
    uint8_t *pool;
    int B, S_max, H_kv, d, page, num_pages, max_blocks;
    size_t page_bytes;          // page * H_kv * d + 4 * page
};

hipError_t launch_kv_quantize_fp8(const KvQuantArgs &a, hipStream_t stream);

// The inverse: token t < len(b) of sequence b is read from row t % page of page
// block_table[b][t / page] of an FP8 pool and written, dequantised, to x [B][S_max][H_kv][d]
// (a page outside the pool gives a zero row; rows at or past len(b) are not written).
struct KvDequantArgs {
    const uint8_t *pool;
    const int32_t *seqlens;     // [B] or nullptr (= S_max)
    const int32_t *block_table; // [B][max_blocks]
    uint16_t *x;
    int B, S_max, H_kv, d, page, num_pages, max_blocks;
    size_t page_bytes;
};

hipError_t launch_kv_dequantize_fp8(const KvDequantArgs &a, hipStream_t stream);

// Partial states to merge for (b, r), r = h * T + i the row of query head h, token i:
//   uniform_tiles > 0 (decode workspace, every sequence of uniform_tiles 16-key tiles):
//     the slots of sequence b follow from the split plan itself -- the partitions x of
//     the B * uniform_tiles tiles cut into W = min(units, B * uniform_tiles) ranges that
//     hold a tile of b, in slot x + b -- at index slot * state_stride + r * head_stride;
//   seg != nullptr (decode workspace): states p < seg[2b+1], at index
//     (seg[2b] + p) * state_stride + r * head_stride;
//   otherwise (caller's partials, T = 1): states p < (counts ? clamp(counts[b], 0, P) : P),
//     at index b * batch_stride + r * head_stride + p * state_stride.
// The O array holds d values per index, bf16 (o_bf16: the decode workspace) or fp32 (the
// caller's partials).  Outputs: o [B][T][H_q][d], lse [B][H_q][T].
struct MergeArgs {
    const float *part_m2, *part_l;
    const void *part_o;
    int o_bf16;
    int uniform_tiles, units;
    const int32_t *seg;         // [B][2] or nullptr
    const int32_t *counts;      // [B] or nullptr
    int P;
    long batch_stride, head_stride, state_stride;
    uint16_t *o;                // bf16 out
    float *lse;
    int B, H_q, d, T;
};

// Causal prefill of T query rows per sequence, row i being token q_start + i (sees keys
// j <= q_start + i), against a cache of S rows per sequence (q_start + T <= S).
// q, o [B][T][H_q][d]; k, v [B][S][H_kv][d]; lse [B][H_q][T].  Whole prompt: T = S, q_start = 0.
struct PrefillArgs {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int B, S, H_q, H_kv, d;
    int T, q_start;
    float scale_log2;
    // Paged cache when block_table is not null: k and v are pools [num_pages][page][H_kv][d]
    // and key t of sequence b is row t % page of page block_table[b * max_blocks + t / page]
    // (page a multiple of 16; at most kPrefillMaxPages blocks of a sequence are visible).
    const int32_t *block_table;
    int page, num_pages, max_blocks;
    // Per-sequence chunk starts (paged, optional): sequence b's rows are the tokens
    // q_starts[b] .. + T - 1, q_starts[b] clamped to [0, q_start_max].
    const int32_t *q_starts;
    int q_start_max;
};

// Blocks of one sequence a paged prefill can see (its table row is staged in LDS).
constexpr int kPrefillMaxPages = 8192;

// Backward of whole-prompt causal prefill: q, o, dout, dq [B][S][H_q][d]; k, v, dk, dv
// [B][S][H_kv][d] (bf16); lse [B][H_q][S] (natural log, the forward's).  The workspace holds
// the per-row statistics (lse in log2 units and D = dO . O per 64-row block).
struct BwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float *stats;                       // set by the launcher: the workspace
    int B, S, H_q, H_kv, d;
    float scale;                        // softmax_scale (tau)
    float scale_log2;                   // tau * log2(e)
};

size_t prefill_bwd_workspace_bytes(int B, int S, int H_q);
hipError_t launch_prefill_bwd(BwdArgs a, void *ws, hipStream_t stream);

// Plain streaming read of `bytes` bytes (a multiple of 16) of device memory; sink holds
// hbm_read_blocks() words and is written only in the (data-dependent, unlikely) case that
// a workgroup's checksum equals the launch's magic value.
int hbm_read_blocks();
hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

// Rounds of independent bf16 32x32x16 matrix products on operands loaded from `ops`
// (`bytes`, a multiple of 16, at least 256 B); sink holds mfma_rate_threads() floats, one
// written per thread.  mfma_rate_flop(iters) is the FLOP count of one launch.
int mfma_rate_threads();
double mfma_rate_flop(int iters);
hipError_t launch_mfma_rate(const void *ops, size_t bytes, int iters, float *sink,
                            hipStream_t stream);

// The library's own decode workspace on the current device (decode_noalloc.hip): its
// size, and its device address (looked up once per device, on first use).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_decode_split(const DecodeSplitArgs &a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs &a, hipStream_t stream);
hipError_t launch_prefill_causal(const PrefillArgs &a, hipStream_t stream);

}  // namespace gqa
