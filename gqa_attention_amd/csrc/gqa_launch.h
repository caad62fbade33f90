// gqa_launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
//
// Every launcher trusts its arguments: the C ABI layer validates shapes,
// pointers and sizes before calling any of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// Split-KV plan: the keys of a sequence are cut into chunks of `chunk` keys (P chunks for
// the longest sequence) and every chunk into `slabs` slabs of `slab` keys (the last ragged).
// One workgroup sweeps one slab for `hpw` KV heads at once, so it reads whole runs of the
// cache's [token][kv head][d] rows; each (query head, chunk, slab) gets one partial state,
// stored state-major: [B][chunk * slabs + slab][H_q] (O: [..][d]), so the states a
// workgroup writes are contiguous.
struct DecodeSplitArgs {
    const uint16_t *q, *k, *v;  // bf16 bit patterns
    const int32_t *seqlens;     // [B] or nullptr
    float *part_m2, *part_l, *part_o;
    int B, H_q, H_kv, d, S_max;
    int chunk, P;               // keys per chunk, chunks of the longest sequence
    int slab, slabs;            // keys per slab, slabs per chunk
    int hpw;                    // KV heads per workgroup (divides H_kv and the wave count)
    float scale_log2;           // softmax_scale * log2(e)
    // Paged cache when block_table is not null: k and v are pools [num_pages][page][H_kv][d]
    // and key t of sequence b is row t % page of page block_table[b * max_blocks + t / page]
    // (page a multiple of 16; S_max = max_blocks * page).
    const int32_t *block_table;
    int page, num_pages, max_blocks;
};

// Partial state (b, h, p) sits at index b*batch_stride + h*head_stride + p*state_stride of
// the m2 and l arrays, and at d times that index in the O array.
struct MergeArgs {
    const float *part_m2, *part_l, *part_o;
    const int32_t *counts;      // [B] or nullptr
    int counts_are_lengths;     // 1: counts are sequence lengths, states = ceil(len/chunk)*slabs
    int chunk, slabs, S_max;    // used when counts_are_lengths
    int P;                      // states per row when counts is nullptr (and the upper bound)
    long batch_stride, head_stride, state_stride;
    uint16_t *o;                // bf16 out [B, H_q, d]
    float *lse;                 // [B, H_q]
    int B, H_q, d;
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
};

hipError_t launch_decode_split(const DecodeSplitArgs &a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs &a, hipStream_t stream);
hipError_t launch_prefill_causal(const PrefillArgs &a, hipStream_t stream);

}  // namespace gqa
