// decode_split.hip -- stage 1 of split-KV decode on gfx950.
//
// The keys of a sequence are cut into chunks and every chunk into slabs.  One
// workgroup per (slab, group of up to 8 KV heads, sequence b) sweeps the slab's
// keys with an online softmax and writes the slab's partial state (m2, l, O) for
// every query head of those KV heads ("Attention Kernel lineage" (V07), section 17: split-K
// partial kernel; section 2: running (m, l, O) update; ADR-0060 "AHBM GQA Fused
// Attention", section 3: per-tile op sequence of the decode sweep).
//
// GQA M-fold (ADR-0060 TL;DR and section 5.2; V07 section 14): the G query heads
// of a KV head share every K/V tile, so each K/V byte is read from HBM once.
// On the matrix cores the product is formed transposed, S^T = K . Q^T, so keys
// are the 16 rows of the MFMA and the (up to 16) query heads its columns: the
// K fragment of a lane is 4 x 16 contiguous bytes of one key row and goes from
// HBM straight into the A operand registers, and each lane ends up owning one
// head's scores, so the softmax row statistics need only two cross-lane steps.
//
// The P.V product is formed as O^T = V^T . P^T: P^T is exactly the S^T registers
// after the softmax (no data movement), and V^T fragments (8 keys of one d
// column per lane) come from a per-wave LDS copy of the V tile through the LDS
// transpose read.
//
// The 8 waves of a workgroup are spread over its KV heads, so at any moment the
// workgroup streams whole [kv head][d] runs of consecutive cache rows (a probe on
// MI355X read this pattern at ~6 TB/s against ~4.9 TB/s when each workgroup
// owned one head's 256-byte slices of a longer key range).  The waves of one head
// take interleaved 32-key tiles (the K-split of V07 section 7/8) with the next
// tile's loads in flight while the current one is computed (ADR-0060 TL;DR,
// software pipelining); with one wave per head the state is written straight
// from registers, otherwise the waves merge through LDS (V07 section 8).
//
// Scores are kept in log2 units: s2 = (q.k) * tau * log2(e), folded into one
// fp32 multiplier applied to the fp32 accumulator (V07 section 2, exp2 trick).
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kTile = 16;   // keys per tile: one 16-row matrix-core tile
constexpr int kDepth = 2;   // tiles in flight per wave
constexpr int kWaves = 8;

template <int D>
struct DecodeTraits {
    static constexpr int KS = D / 32;           // 32-deep k-steps of Q.K^T
    static constexpr int LPR = D / 8;           // lanes per V row (16 B each)
    static constexpr int RPI = 64 / LPR;        // V rows per wave load
    static constexpr int NVI = kTile / RPI;     // V loads per lane per tile
    static constexpr int NDT = D / 16;          // 16-wide d tiles of O^T
    static constexpr int VPITCH = D + 16;       // staged V row pitch (bf16): 16-B aligned,
                                                // 4 consecutive rows on disjoint banks
};

template <int D>
struct TileRegs {
    u32x4 k[DecodeTraits<D>::KS];
    u32x4 v[DecodeTraits<D>::NVI];
};

// Per-lane byte offsets of a tile's loads from the tile's first key row (loop invariant).
template <int D>
struct TileOffsets {
    uint32_t k;                               // K: row lane%16, d-slots from 8*(lane/16)*KS
    uint32_t v[DecodeTraits<D>::NVI];         // V: row i*RPI + lane/LPR, 16 B at lane%LPR
};

// Load a 16-key tile of one KV head whose first key row (that head's slice of it) sits at
// kt / vt, with the following rows kv_row elements apart.  Only the first `bytes` bytes
// from kt / vt are read; the rest of the tile reads as zeros and costs no memory traffic,
// so a tile that lies wholly past the end (bytes = 0) may be "loaded" unconditionally.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &r, const uint16_t *kt, const uint16_t *vt,
                                          uint32_t bytes, const TileOffsets<D> &off) {
    using T = DecodeTraits<D>;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt, bytes);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) r.k[ks] = buffer_load16(rk, off.k, ks * 16);
#pragma unroll
    for (int i = 0; i < T::NVI; ++i) r.v[i] = buffer_load16(rv, off.v[i], 0);
}

// Lazy-rescale slack in log2 units: the shared running max moves only when a score
// passes it by more than this, so P <= 2^kSlack in between (exact: a common shift
// cancels in O / l, V07 section 3).
constexpr float kSlack = 8.f;

template <int D>
struct WaveState {
    float m;                          // running max shared by the 4 lanes of a head (log2 units)
    float l;                          // this lane's share of the denominator (fp32 P)
    float lw;                         // the same from the bf16-rounded P that enters P.V
    f32x4 o[DecodeTraits<D>::NDT];    // O^T tiles: d = 16*dt + 4*grp + r, head = lane%16
};

// First half of a tile: S^T = K . Q^T (rows: keys key0 + 4*(lane/16) + r, column: head
// lane%16) and the V tile staged row-major in the wave's LDS area.  After it the tile's
// registers are free for the next prefetch.
template <int D>
__device__ __forceinline__ f32x4 score_tile(const TileRegs<D> &r,
                                            const bf16x8 (&qf)[DecodeTraits<D>::KS],
                                            uint16_t *vs, int lane) {
    using T = DecodeTraits<D>;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) s = mfma16(as_bf16x8(r.k[ks]), qf[ks], s);
#pragma unroll
    for (int i = 0; i < T::NVI; ++i) {
        uint16_t *dst = vs + (i * T::RPI + lane / T::LPR) * T::VPITCH + (lane % T::LPR) * 8;
        *reinterpret_cast<u32x4 *>(dst) = r.v[i];
    }
    return s;
}

// Second half: online softmax of the tile's scores and O^T += V^T . P^T.
template <int D>
__device__ __forceinline__ void softmax_pv(WaveState<D> &st, f32x4 s, const uint16_t *vs,
                                           int key0, int key_end, float scale_log2, int lane) {
    using T = DecodeTraits<D>;
    const int row16 = lane & 15, grp = lane >> 4;

    // scale to log2 units; keys past the slab/sequence end are masked
    float s2[4];
    float mx = neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x = key0 + grp * 4 + i < key_end ? s[i] * scale_log2 : neg_inf();
        s2[i] = x;
        mx = fmaxf(mx, x);
    }
    // Each lane holds 4 of a head's 16 scores.  Only when one of them passes the shared
    // max by the slack (always on the first tile, where m = -inf) do the head's 4 lanes
    // agree on a new max and rescale; otherwise no cross-lane step is needed.
    if (__any(mx > st.m + kSlack)) {
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float m_new = fmaxf(st.m, mx);
        const float alpha = exp2_fast(st.m - m_new);   // 0 on the first tile
        st.l *= alpha;
        st.lw *= alpha;
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt) st.o[dt] *= alpha;
        st.m = m_new;
    }

    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        p[j] = exp2_fast(s2[j] - st.m);
        st.l += p[j];
    }
    // P^T as the B operand of the 16x16x16 product: keys 4*grp + j, head lane%16
    const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    const s16x4 pf = __builtin_bit_cast(s16x4, pw);
    st.lw = add_bf16_pair(pw[0], st.lw);
    st.lw = add_bf16_pair(pw[1], st.lw);

    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T.  V^T fragment of lane (row16, grp): column d = 16*dt + row16,
    // keys 4*grp + 0..3, via one LDS transpose read whose lanes point at row
    // 4*grp + row16/4, columns 16*dt + 4*(row16%4).
    const uint16_t *vrow = vs + (4 * grp + (row16 >> 2)) * T::VPITCH + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) {
        const s16x4 vf = __builtin_bit_cast(s16x4, lds_read_tr16(vrow + dt * 16));
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, st.o[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

// End of a wave's sweep: add up the head's four lane shares of l and lw, and scale O^T
// by l / lw so that O / l is the convex combination of V with the rounded weights.
template <int D>
__device__ __forceinline__ void finish_state(WaveState<D> &st) {
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    st.lw += __shfl_xor(st.lw, 16);
    st.lw += __shfl_xor(st.lw, 32);
    const float f = st.lw > 0.f ? st.l / st.lw : 0.f;
#pragma unroll
    for (int dt = 0; dt < DecodeTraits<D>::NDT; ++dt) st.o[dt] *= f;
}

// Paged: the cache is a pool of pages of a.page consecutive key rows ([page][row][H_kv][d]),
// and key t of sequence b is row t % page of page block_table[b][t / page] (V07 section
// 16, logical token to page map; section 17, the decode kernel reads through the table).
// Chunks and slabs start at multiples of 32 keys and a page holds a multiple of 16, so a
// 16-key tile never crosses a page: each tile is one table lookup plus the contiguous
// read of the unpaged cache.  The lookups of a wave's tiles (at most 8 of them) are
// loaded once, one per lane, before the sweep (the table is read when the workgroup
// starts, as V07 section 17 describes), and each tile takes its entry with a lane read.
template <int D, bool Paged>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(DecodeSplitArgs a, int n_hg) {
    using T = DecodeTraits<D>;
    // V staging during the sweep, then (several waves per head) the cross-wave merge
    constexpr int kStageBytes = kWaves * kTile * T::VPITCH * 2;
    constexpr int kMergeBytes = kWaves * 16 * (D + 2) * 4;
    __shared__ __attribute__((aligned(16)))
    uint16_t smem[(kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes) / 2];

    const int p = blockIdx.x / a.slabs, sl = blockIdx.x % a.slabs;
    const int hgrp = blockIdx.y / n_hg, hg = blockIdx.y % n_hg;
    const int b = blockIdx.z;
    const int G = a.H_q / a.H_kv;
    const int Sb = a.seqlens ? min(max(a.seqlens[b], 0), a.S_max) : a.S_max;
    const int c0 = p * a.chunk;
    if (c0 >= Sb) return;  // the whole chunk is past the sequence end: its states are never read
    const int c1 = min(c0 + a.chunk, Sb);
    const int s0 = c0 + sl * a.slab;
    const int s1 = min(s0 + a.slab, c1);

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row16 = lane & 15, grp = lane >> 4;
    // wave w sweeps KV head hw of this workgroup's group; the wph waves of one head take
    // interleaved 16-key tiles of the slab (phase = first tile)
    const int wph = kWaves / a.hpw;
    const int hw = w % a.hpw, phase = w / a.hpw;
    const int hk = hgrp * a.hpw + hw;
    const int h0 = hk * G + hg * 16;
    const int nh = min(16, G - hg * 16);
    // this slab's states: [b][state][H_q], state = p * slabs + sl
    const size_t n_states = (size_t)a.P * a.slabs;
    const size_t srow = ((size_t)b * n_states + (size_t)p * a.slabs + sl) * a.H_q;

    if (s0 >= s1) {  // a slab past the end of a live chunk: mark its states empty
        if (phase == 0 && lane < nh) {
            a.part_m2[srow + h0 + lane] = neg_inf();
            a.part_l[srow + h0 + lane] = 0.f;
        }
        return;
    }

    // Q^T fragments (B operand): column = query head h0 + row16, k-slots = d.  Columns past
    // the group's last head repeat that head; their results are never stored.
    bf16x8 qf[T::KS];
    {
        const uint16_t *qrow =
            a.q + ((size_t)b * a.H_q + h0 + min(row16, nh - 1)) * D + grp * (D / 4);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) qf[ks] = as_bf16x8(load16(qrow + ks * 8));
    }

    const size_t kv_row = (size_t)a.H_kv * D;
    // unpaged: this sequence's cache, head hk; paged: the pool, head hk
    const size_t head_off = Paged ? (size_t)hk * D : ((size_t)b * a.S_max * a.H_kv + hk) * D;
    const uint16_t *kbase = a.k + head_off;
    const uint16_t *vbase = a.v + head_off;
    uint16_t *vs = smem + w * kTile * T::VPITCH;

    WaveState<D> st;
    st.m = neg_inf();
    st.l = 0.f;
    st.lw = 0.f;
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This wave's tiles are phase, phase + wph, ...; tile t starts at key0(t).  kDepth tiles
    // are in flight in a ring of register sets: as soon as tile t's scores are formed and
    // its V is staged, tile t + kDepth is loaded into the freed set, before the softmax and
    // P.V of tile t.  Tiles past the end read zeros without touching memory, so every
    // iteration issues the same loads and the load counter only drains the oldest tile.
    const int ntiles = (s1 - s0 + kTile - 1) / kTile;
    const int n_w = phase < ntiles ? (ntiles - 1 - phase) / wph + 1 : 0;
    TileOffsets<D> toff;
    toff.k = (uint32_t)((row16 * kv_row + grp * (D / 4)) * 2);
#pragma unroll
    for (int i = 0; i < T::NVI; ++i)
        toff.v[i] = (uint32_t)(((i * T::RPI + lane / T::LPR) * kv_row + (lane % T::LPR) * 8) * 2);
    auto key0 = [&](int t) { return s0 + (phase + t * wph) * kTile; };
    // Paged: lane t holds the pool row of this wave's tile t (-1: no tile, or a table
    // entry outside the pool, which then reads as zeros instead of faulting).
    int prow = -1;
    if constexpr (Paged) {
        if (lane < n_w) {
            const int key = key0(lane);
            const int pg = a.block_table[(size_t)b * a.max_blocks + key / a.page];
            if ((unsigned)pg < (unsigned)a.num_pages) prow = pg * a.page + key % a.page;
        }
    }
    // Tile t of this wave: the address of its first row (in kt, vt) and the bytes that
    // hold live keys (rows at or past the slab end read as zeros).
    // (All of it is uniform; readfirstlane keeps the buffer resources in scalar registers.)
    auto issue = [&](TileRegs<D> &r, int t) {
        const int k0 = key0(t);
        if constexpr (Paged) {
            const int pr = __builtin_amdgcn_readlane(prow, t & 63);
            const uint32_t live = (uint32_t)min(max(s1 - k0, 0), kTile);
            const size_t row = (size_t)max(pr, 0) * kv_row;
            const uint32_t bytes = __builtin_amdgcn_readfirstlane(
                pr >= 0 ? live * (uint32_t)kv_row * 2u : 0u);
            load_tile<D>(r, kbase + row, vbase + row, bytes, toff);
        } else {
            const size_t row = (size_t)k0 * kv_row;
            load_tile<D>(r, kbase + row, vbase + row,
                         (uint32_t)max(s1 - k0, 0) * (uint32_t)kv_row * 2u, toff);
        }
    };
    TileRegs<D> ring[kDepth];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
        issue(ring[j], j);
        __builtin_amdgcn_sched_barrier(0);   // keep the ring's issue order: oldest tile first
    }
    // whole rounds of kDepth tiles (no exit inside a round, so every pass through the loop
    // has the same loads outstanding), then the last n_w % kDepth tiles with no new loads
    const int n_full = n_w - n_w % kDepth;
    int t = 0;
    for (; t < n_full; t += kDepth) {
#pragma unroll
        for (int j = 0; j < kDepth; ++j) {
            const f32x4 sc = score_tile<D>(ring[j], qf, vs, lane);
            __builtin_amdgcn_sched_barrier(0);
            issue(ring[j], t + j + kDepth);
            softmax_pv<D>(st, sc, vs, key0(t + j), s1, a.scale_log2, lane);
        }
    }
#pragma unroll
    for (int j = 0; j < kDepth - 1; ++j) {
        if (t + j >= n_w) break;
        const f32x4 sc = score_tile<D>(ring[j], qf, vs, lane);
        softmax_pv<D>(st, sc, vs, key0(t + j), s1, a.scale_log2, lane);
    }

    finish_state<D>(st);

    if (wph == 1) {
        // one wave per head: its registers hold the slab's whole state
        if (row16 < nh) {
            const size_t row = srow + h0 + row16;
            float *orow = a.part_o + row * D + grp * 4;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) *reinterpret_cast<f32x4 *>(orow + dt * 16) = st.o[dt];
            if (grp == 0) {
                a.part_m2[row] = st.m;
                a.part_l[row] = st.l;
            }
        }
        return;
    }

    // several waves per head: merge their states through LDS (reusing the V staging area):
    // red[w][head][0..D) = O^T column, [D] = m, [D+1] = l
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
    constexpr int RS = D + 2;
    float *mine = red + (w * 16 + row16) * RS;
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[dt * 16 + grp * 4 + i] = st.o[dt][i];
    if (grp == 0) {
        mine[D] = st.m;
        mine[D + 1] = st.l;
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < a.hpw * nh * D; idx += kWaves * 64) {
        const int hw2 = idx / (nh * D), h = (idx / D) % nh, d = idx % D;
        float M = neg_inf();
        for (int ph = 0; ph < wph; ++ph) M = fmaxf(M, red[((hw2 + a.hpw * ph) * 16 + h) * RS + D]);
        float L = 0.f, O = 0.f;
        for (int ph = 0; ph < wph; ++ph) {
            const float *rw = red + ((hw2 + a.hpw * ph) * 16 + h) * RS;
            const float al = exp2_fast(rw[D] - M);  // a wave without tiles: 2^-inf = 0
            L += al * rw[D + 1];
            O += al * rw[d];
        }
        const int hk2 = hgrp * a.hpw + hw2;
        const size_t row = srow + hk2 * G + hg * 16 + h;
        a.part_o[row * D + d] = O;
        if (d == 0) {
            a.part_m2[row] = M;
            a.part_l[row] = L;
        }
    }
}

template <int D>
hipError_t launch(const DecodeSplitArgs &a, hipStream_t stream) {
    const int G = a.H_q / a.H_kv;
    const int n_hg = (G + 15) / 16;
    dim3 grid(a.P * a.slabs, (a.H_kv / a.hpw) * n_hg, a.B);
    if (a.block_table)
        hipLaunchKernelGGL((decode_split_kernel<D, true>), grid, dim3(kWaves * 64), 0, stream, a,
                           n_hg);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, false>), grid, dim3(kWaves * 64), 0, stream, a,
                           n_hg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeSplitArgs &a, hipStream_t stream) {
    switch (a.d) {
    case 32: return launch<32>(a, stream);
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gqa
