// decode_split.hip -- stage 1 of split-KV decode on gfx950.
//
// Every sequence's keys are cut into 16-key tiles, and the tiles of all the
// sequences of the batch, taken in order, into W equal contiguous partitions,
// one per workgroup (W is about one per compute unit).  A workgroup sweeps its
// partition with an online softmax for a group of up to 8 KV heads and, each
// time its partition leaves a sequence, writes that sequence's partial state
// (m2, l, O) for every query head of those KV heads ("Attention Kernel lineage"
// (V07), section 17: split-K partial kernel, partitions of the key axis;
// section 2: running (m, l, O) update; ADR-0060 "AHBM GQA Fused Attention",
// section 3: per-tile op sequence of the decode sweep).  So the work is split
// evenly however ragged the lengths are, a workgroup streams without a break
// from its first tile to its last (the next tile's loads are issued before a
// finished state is stored), and a sequence gets one state per workgroup that
// touches it -- about W + B states per query head for the whole batch.
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
// owned one head's 256-byte slices of a longer key range).  With fewer KV heads
// than waves, the waves of one head take interleaved tiles (the K-split of V07
// sections 7-8) and merge their states through LDS before a state is written.
// Each wave keeps the next tile's loads in flight while it computes the current
// one (ADR-0060 TL;DR, software pipelining).
//
// Scores are kept in log2 units: s2 = (q.k) * tau * log2(e), folded into one
// fp32 multiplier applied to the fp32 accumulator (V07 section 2, exp2 trick).
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kTile = 16;      // keys per tile: one 16-row matrix-core tile
constexpr int kWaves = 8;
constexpr int kWindow = 64;    // paged: table lookups fetched at once, one per lane

template <int D>
struct DecodeTraits {
    static constexpr int KS = D / 32;           // 32-deep k-steps of Q.K^T
    static constexpr int LPR = D / 8;           // lanes per V row (16 B each)
    static constexpr int RPI = 64 / LPR;        // V rows per wave load
    static constexpr int NVI = kTile / RPI;     // V loads per lane per tile
    static constexpr int NDT = D / 16;          // 16-wide d tiles of O^T
    static constexpr int VPITCH = D + 16;       // staged V row pitch (bf16): 16-B aligned,
                                                // 4 consecutive rows on disjoint banks
    // FP8 pages: rows of D one-byte codes
    static constexpr int LPR8 = D / 16;         // lanes per V row (16 codes each)
    static constexpr int RPI8 = 64 / LPR8;      // V rows per wave load
    static constexpr int NVI8 = kTile / RPI8;   // V loads per lane per tile
};

template <int D, bool Fp8>
struct TileRegs {
    u32x4 k[DecodeTraits<D>::KS];
    u32x4 v[DecodeTraits<D>::NVI];
};

// FP8 pages: the lane's 8 * KS K codes (the same key row and d-slots as the bf16 tile, in
// half the bytes), its share of the V tile's codes, and the fp32 per-token scales of the
// lane's four keys 4*(lane/16) .. +3 for K (its scores) and for V (its P values).
template <int D>
struct TileRegs<D, true> {
    u32x4 k[DecodeTraits<D>::KS / 2];
    u32x4 v[DecodeTraits<D>::NVI8];
    u32x4 ksc, vsc;
};

// Per-lane byte offsets of a tile's loads from the tile's first key row (loop invariant).
template <int D>
struct TileOffsets {
    uint32_t k;                               // K: row lane%16, d-slots from 8*(lane/16)*KS
    uint32_t v[DecodeTraits<D>::NVI];         // V: row i*RPI + lane/LPR, 16 B at lane%LPR
};

template <int D>
struct TileOffsets8 {
    uint32_t k;                               // K codes: row lane%16, byte (lane/16) * D/4
    uint32_t v[DecodeTraits<D>::NVI8];        // V codes: row i*RPI8 + lane/LPR8, 16 B at lane%LPR8
};

// Eight E4M3 codes (two dwords, lowest byte first) as eight bf16 values: exact, since every
// E4M3 value is a bfloat16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// FP8 tile: codes of 16 key rows from kt / vt (rows row_bytes apart; `bytes` of them real)
// and the per-token scales from kst / vst (`sbytes` real); the rest reads as zeros.
template <int D>
__device__ __forceinline__ void load_tile8(TileRegs<D, true> &r, const uint8_t *kt,
                                           const uint8_t *vt, const uint8_t *kst, const uint8_t *vst,
                                           uint32_t bytes, uint32_t sbytes,
                                           const TileOffsets8<D> &off, int grp) {
    using T = DecodeTraits<D>;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt, bytes);
#pragma unroll
    for (int j = 0; j < T::KS / 2; ++j) r.k[j] = buffer_load16(rk, off.k, j * 16);
#pragma unroll
    for (int i = 0; i < T::NVI8; ++i) r.v[i] = buffer_load16(rv, off.v[i], 0);
    r.ksc = buffer_load16(make_rsrc(kst, sbytes), 16u * (uint32_t)grp, 0);
    r.vsc = buffer_load16(make_rsrc(vst, sbytes), 16u * (uint32_t)grp, 0);
}

// Load a 16-key tile of one KV head whose first key row (that head's slice of it) sits at
// kt / vt, with the following rows kv_row elements apart.  Only the first `bytes` bytes
// from kt / vt are read; the rest of the tile reads as zeros and costs no memory traffic,
// so a tile that lies wholly past the end (bytes = 0) may be "loaded" unconditionally.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D, false> &r, const uint16_t *kt, const uint16_t *vt,
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
// Running max before a column's first live key: finite, so that 2^(kNoMax - kNoMax) = 1
// and 2^(-inf - kNoMax) = 0 (no -inf - -inf); a state that never saw a live key is
// stored with m2 = -inf, the empty state of the merge.
constexpr float kNoMax = -1e30f;

// A wave's running state for its CB blocks of 16 columns.
template <int D, int CB>
struct WaveState {
    float m[CB];                         // running max shared by a column's 4 lanes (log2 units)
    float l[CB];                         // this lane's share of the denominator (fp32 P)
    float lw[CB];                        // the same from the bf16-rounded P that enters P.V
    f32x4 o[CB][DecodeTraits<D>::NDT];   // O^T tiles: d = 16*dt + 4*grp + r, column lane%16
};

// First half of a tile: S^T = K . Q^T for each block of 16 columns (rows: keys key0 +
// 4*(lane/16) + r, column lane%16 of the block), sharing each K fragment, and the V tile
// staged row-major in the wave's LDS area.  After it the tile's registers are free for the
// next prefetch.
template <int D, int CB>
__device__ __forceinline__ void score_tile(const TileRegs<D, false> &r,
                                           const bf16x8 (&qf)[CB][DecodeTraits<D>::KS],
                                           uint16_t *vs, int lane, f32x4 (&s)[CB]) {
    using T = DecodeTraits<D>;
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) s[bk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
        for (int bk = 0; bk < CB; ++bk) s[bk] = mfma16(as_bf16x8(r.k[ks]), qf[bk][ks], s[bk]);
#pragma unroll
    for (int i = 0; i < T::NVI; ++i) {
        uint16_t *dst = vs + (i * T::RPI + lane / T::LPR) * T::VPITCH + (lane % T::LPR) * 8;
        *reinterpret_cast<u32x4 *>(dst) = r.v[i];
    }
}

// The same from FP8 codes: K and V converted to bf16 in registers (exactly) in the order of
// the bf16 path, V staged as bf16 rows; the scores still lack the per-token K scale.
template <int D, int CB>
__device__ __forceinline__ void score_tile8(const TileRegs<D, true> &r,
                                            const bf16x8 (&qf)[CB][DecodeTraits<D>::KS],
                                            uint16_t *vs, int lane, f32x4 (&s)[CB]) {
    using T = DecodeTraits<D>;
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) s[bk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < T::KS / 2; ++j) {
        const bf16x8 k0 = e4m3x8_to_bf16(r.k[j][0], r.k[j][1]);
        const bf16x8 k1 = e4m3x8_to_bf16(r.k[j][2], r.k[j][3]);
#pragma unroll
        for (int bk = 0; bk < CB; ++bk) s[bk] = mfma16(k0, qf[bk][2 * j], s[bk]);
#pragma unroll
        for (int bk = 0; bk < CB; ++bk) s[bk] = mfma16(k1, qf[bk][2 * j + 1], s[bk]);
    }
#pragma unroll
    for (int i = 0; i < T::NVI8; ++i) {
        uint16_t *dst = vs + (i * T::RPI8 + lane / T::LPR8) * T::VPITCH + (lane % T::LPR8) * 16;
        *reinterpret_cast<bf16x8 *>(dst) = e4m3x8_to_bf16(r.v[i][0], r.v[i][1]);
        *reinterpret_cast<bf16x8 *>(dst + 8) = e4m3x8_to_bf16(r.v[i][2], r.v[i][3]);
    }
}

// Second half: online softmax of the tile's scores and O^T += V^T . P^T, for each block
// of columns.  key_end[bk] is this lane's column's bound: its query sees keys below it.
// FP8 pages: ksc / vsc are the per-token scales of the lane's four keys; a score is scaled
// by its key's K scale, and P by its key's V scale on its way into the P.V product (the row
// sums keep the unscaled P).  With power-of-two scales both are exact, so the result equals
// that of bf16 pages holding the dequantised values.
template <int D, int CB, bool Fp8>
__device__ __forceinline__ void softmax_pv(WaveState<D, CB> &st, const f32x4 (&s)[CB],
                                           const uint16_t *vs, int key0, const int (&key_end)[CB],
                                           float scale_log2, int lane, const float (&ksc)[4],
                                           const float (&vsc)[4]) {
    using T = DecodeTraits<D>;
    const int row16 = lane & 15, grp = lane >> 4;
    s16x4 pf[CB];
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) {
        // scale to log2 units; keys at or past the column's bound are masked
        float s2[4];
        float mx = neg_inf();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float c = Fp8 ? scale_log2 * ksc[i] : scale_log2;
            const float x = key0 + grp * 4 + i < key_end[bk] ? s[bk][i] * c : neg_inf();
            s2[i] = x;
            mx = fmaxf(mx, x);
        }
        // Each lane holds 4 of a column's 16 scores.  Only when one of them passes the
        // shared max by the slack (always on the first live key, as m starts at kNoMax) do
        // the column's 4 lanes agree on a new max and rescale; otherwise no cross-lane step
        // is needed.  A column with no live key yet keeps m = kNoMax, so its alpha is 1 and
        // its P is 0 when another column moves the wave into the rescale.
        if (__any(mx > st.m[bk] + kSlack)) {
            mx = wave_max_xor(mx, 16);
            mx = wave_max_xor(mx, 32);
            const float m_new = fmaxf(st.m[bk], mx);
            const float alpha = exp2_fast(st.m[bk] - m_new);   // 0 on a column's first live key
            st.l[bk] *= alpha;
            st.lw[bk] *= alpha;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) st.o[bk][dt] *= alpha;
            st.m[bk] = m_new;
        }

        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = exp2_fast(s2[j] - st.m[bk]);
            st.l[bk] += p[j];
        }
        // P^T as the B operand of the 16x16x16 product: keys 4*grp + j, column lane%16
        const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        if constexpr (Fp8) {
            const u32x2 pv = {pack_bf16x2(p[0] * vsc[0], p[1] * vsc[1]),
                              pack_bf16x2(p[2] * vsc[2], p[3] * vsc[3])};
            pf[bk] = __builtin_bit_cast(s16x4, pv);
        } else {
            pf[bk] = __builtin_bit_cast(s16x4, pw);
        }
        st.lw[bk] = add_bf16_pair(pw[0], st.lw[bk]);
        st.lw[bk] = add_bf16_pair(pw[1], st.lw[bk]);
    }

    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T.  V^T fragment of lane (row16, grp): column d = 16*dt + row16,
    // keys 4*grp + 0..3, via one LDS transpose read whose lanes point at row
    // 4*grp + row16/4, columns 16*dt + 4*(row16%4); one read serves every block.
    const uint16_t *vrow = vs + (4 * grp + (row16 >> 2)) * T::VPITCH + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) {
        const s16x4 vf = __builtin_bit_cast(s16x4, lds_read_tr16(vrow + dt * 16));
#pragma unroll
        for (int bk = 0; bk < CB; ++bk)
            st.o[bk][dt] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf[bk], st.o[bk][dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

// End of a state: add up each column's four lane shares of l and lw, and scale O^T by
// l / lw so that O / l is the convex combination of V with the rounded weights; a column
// that saw no live key gets the empty state (m2 = -inf).
template <int D, int CB>
__device__ __forceinline__ void finish_state(WaveState<D, CB> &st) {
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) {
        st.l[bk] += __shfl_xor(st.l[bk], 16);
        st.l[bk] += __shfl_xor(st.l[bk], 32);
        st.lw[bk] += __shfl_xor(st.lw[bk], 16);
        st.lw[bk] += __shfl_xor(st.lw[bk], 32);
        const float f = st.lw[bk] > 0.f ? st.l[bk] / st.lw[bk] : 0.f;
#pragma unroll
        for (int dt = 0; dt < DecodeTraits<D>::NDT; ++dt) st.o[bk][dt] *= f;
        if (!(st.l[bk] > 0.f)) st.m[bk] = neg_inf();
    }
}

// Length of sequence b as the kernel uses it: seqlens[b] clamped to [0, S_max].
__device__ __forceinline__ int seq_len(const DecodeSplitArgs &a, int b) {
    return a.seqlens ? min(max(a.seqlens[b], 0), a.S_max) : a.S_max;
}

// Q^T fragments (B operand) of sequence b: column row16 of this wave's 16-column group is
// query row (g, i) = (head hk * G + g, token i) of the G * T rows folded for KV head hk
// (q is [B][T][H_q][d]); k-slots = d.  Columns past the group's last row repeat that row;
// their results are never stored.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DecodeTraits<D>::KS], const DecodeSplitArgs &a,
                                       int b, int hk, int G, int col, int grp) {
    const int g = col / a.T, i = col % a.T;
    const uint16_t *qrow =
        a.q + (((size_t)b * a.T + i) * a.H_q + hk * G + g) * D + grp * (D / 4);
#pragma unroll
    for (int ks = 0; ks < DecodeTraits<D>::KS; ++ks) qf[ks] = as_bf16x8(load16(qrow + ks * 8));
}

// Paged: the cache is a pool of pages of a.page consecutive key rows ([page][row][H_kv][d]),
// and key t of sequence b is row t % page of page block_table[b][t / page] (V07 section
// 16, logical token to page map; section 17, the decode kernel reads through the table).
// Tiles start at multiples of 16 keys and a page holds a multiple of 16, so a tile never
// crosses a page: each tile is one table lookup plus the contiguous read of the unpaged
// cache.  A wave fetches the lookups of its next 64 tiles at once, one per lane (the table
// is read ahead of the sweep, as V07 section 17 describes), and each tile takes its entry
// with a lane read.
//
// A wave folds CB blocks of 16 columns (CB = 2 when a KV head has more than 16 rows, G * T
// > 16), so up to 32 rows share each K fragment, V^T fragment and tile load.
//
// FP8 pages (Fp8, paged only): the pools are byte pools of pages of a.page_bytes bytes --
// a.page rows of [H_kv][D] E4M3 codes, then the page's a.page fp32 per-token scales
// (V07 section 17.7) -- read in half the bytes and dequantised in registers.
template <int D, bool Paged, int CB, bool Fp8>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(DecodeSplitArgs a, int n_hg) {
    using T = DecodeTraits<D>;
    // V staging during the sweep; at a state boundary (several waves per head) the
    // cross-wave merge
    constexpr int kStageBytes = kWaves * kTile * T::VPITCH * 2;
    constexpr int kMergeBytes = kWaves * 16 * (D + 2) * 4;
    __shared__ __attribute__((aligned(16)))
    uint16_t smem[(kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes) / 2];
    __shared__ int32_t pre[kMaxDecodeBatch + 1];   // pre[b]: tiles of sequences 0 .. b-1
    __shared__ uint8_t last[kMaxDecodeBatch];      // keys in sequence b's last tile (1..16)

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row16 = lane & 15, grp = lane >> 4;
    const int G = a.H_q / a.H_kv;
    const int GT = G * a.T;                 // rows folded per KV head: G heads x T tokens
    const int hgrp = blockIdx.y / n_hg, hg = blockIdx.y % n_hg;
    // wave w sweeps KV head hw of this workgroup's group; the wph waves of one head take
    // interleaved tiles of the partition (phase = first tile)
    const int wph = kWaves / a.hpw;
    const int hw = w % a.hpw, phase = w / a.hpw;
    const int hk = hgrp * a.hpw + hw;
    constexpr int CW = 16 * CB;             // columns (rows of the KV head) per wave
    const int h0 = hk * GT + hg * CW;      // first state row of this wave's columns
    // block bk: nhb[bk] live columns (<= 0: none; its lanes repeat the last row and are
    // never stored); this lane's column (g, token) and the tokens after its token
    int nhb[CB], colb[CB], gapb[CB];
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) {
        nhb[bk] = min(16, GT - hg * CW - bk * 16);
        colb[bk] = min(hg * CW + bk * 16 + row16, GT - 1);
        gapb[bk] = a.T - 1 - colb[bk] % a.T;
    }

    // ---- running tile counts of the sequences ----
    // Up to 64 sequences: every wave scans them in its own registers (lane b holds
    // pre[b + 1] and last[b]), with no LDS and no barrier; more: wave 0 scans them into LDS.
    const bool small = a.B <= 64;
    int incl = 0, lastv = 0;
    if (small) {
        const int len = lane < a.B ? seq_len(a, lane) : 0;
        incl = (len + kTile - 1) / kTile;
        lastv = len - (incl - 1) * kTile;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int x = __shfl_up(incl, off);
            if (lane >= off) incl += x;
        }
    } else {
        if (w == 0) {
            int carry = 0;
            if (lane == 0) pre[0] = 0;
            for (int base = 0; base < a.B; base += 64) {
                const int b = base + lane;
                const int len = b < a.B ? seq_len(a, b) : 0;
                int n = (len + kTile - 1) / kTile;
                if (b < a.B) last[b] = (uint8_t)(len - (n - 1) * kTile);
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int x = __shfl_up(n, off);
                    if (lane >= off) n += x;
                }
                if (b < a.B) pre[b + 1] = carry + n;
                carry += __shfl(n, 63);
            }
        }
        __syncthreads();
    }

    // pre[i] for a uniform i (scalar register), and for a per-lane i
    auto P = [&](int i) {
        return small ? (i == 0 ? 0 : __builtin_amdgcn_readlane(incl, i - 1))
                     : __builtin_amdgcn_readfirstlane(pre[i]);
    };
    auto P_lane = [&](int i) {
        const int v = small ? __shfl(incl, max(i - 1, 0)) : pre[i];
        return i == 0 ? 0 : v;
    };
    // length of sequence b (which has tiles [lo, hi), hi > lo)
    auto L = [&](int b, int lo, int hi) {
        const int lt = small ? __builtin_amdgcn_readlane(lastv, b)
                             : __builtin_amdgcn_readfirstlane((int)last[b]);
        return (hi - lo - 1) * kTile + lt;
    };

    // ---- this workgroup's partition [t0, t1) of the batch's tiles ----
    // W partitions, no more than there are tiles, so that none is empty: then the
    // partitions that touch a sequence are consecutive and each holds a state of it
    const int tot = P(a.B);
    const int W = min((int)gridDim.x, tot), x = blockIdx.x;
    // workgroup (0, 0) records where each sequence's states are for the merge: partition
    // x holds its state of sequence b in slot x + b (unique: partitions advance with b)
    if (blockIdx.x == 0 && blockIdx.y == 0 && (!small || w == 0)) {
        for (int b = small ? lane : threadIdx.x; b < (small ? 64 : a.B); b += kWaves * 64) {
            const int lo = P_lane(b), hi = P_lane(b + 1);
            int first = 0, n = 0;
            if (hi > lo) {
                const int x0 = (int)((long)lo * W / tot), x1 = (int)((long)(hi - 1) * W / tot);
                first = x0 + b;
                n = x1 - x0 + 1;
            }
            if (b < a.B) {
                a.seg[2 * b] = first;
                a.seg[2 * b + 1] = n;
            }
        }
    }
    if (x >= W) return;     // no tiles left for this workgroup
    const int t0 = (int)(((long)x * tot + W - 1) / W);
    const int t1 = (int)(((long)(x + 1) * tot + W - 1) / W);

    // the sequence holding tile t0: the last b with pre[b] <= t0 (it has tiles)
    int cb = 0;
    {
        int hi = a.B - 1;
        while (cb < hi) {
            const int mid = (cb + hi + 1) >> 1;
            if (P(mid) <= t0) cb = mid;
            else hi = mid - 1;
        }
    }

    const size_t kv_row = (size_t)a.H_kv * D;
    // unpaged: sequence 0's cache, head hk (plus b * S_max rows per sequence); paged: the
    // pool, head hk
    const uint16_t *kbase = a.k + (size_t)hk * D;
    const uint16_t *vbase = a.v + (size_t)hk * D;
    uint16_t *vs = smem + w * kTile * T::VPITCH;

    TileOffsets<D> toff;
    toff.k = (uint32_t)((row16 * kv_row + grp * (D / 4)) * 2);
#pragma unroll
    for (int i = 0; i < T::NVI; ++i)
        toff.v[i] = (uint32_t)(((i * T::RPI + lane / T::LPR) * kv_row + (lane % T::LPR) * 8) * 2);
    TileOffsets8<D> toff8;                     // FP8: byte offsets, rows kv_row bytes apart
    toff8.k = (uint32_t)(row16 * kv_row + grp * (D / 4));
#pragma unroll
    for (int i = 0; i < T::NVI8; ++i)
        toff8.v[i] = (uint32_t)((i * T::RPI8 + lane / T::LPR8) * kv_row + (lane % T::LPR8) * 16);

    // ---- issue side: the next tile this wave loads, and its sequence ----
    int it = t0 + phase;                       // flattened tile index
    int ib = cb, ilo = P(cb), ihi = P(cb + 1), ilen = L(cb, ilo, ihi);
    int issued = 0;                            // tiles issued by this wave (paged windows)
    int pw = -1;                               // paged: pool row of window tile `lane`
    int ppg = -1, prw = 0;                     // FP8: its page and row within the page
    // Load tile `it` into r (past the partition end: zero bytes, no memory traffic).  All of
    // it is uniform; readfirstlane keeps the buffer resources in scalar registers.
    auto issue = [&](TileRegs<D, Fp8> &r) {
        uint32_t bytes = 0, nkeys = 0;
        size_t row = 0;
        if (it < t1) {
            while (it >= ihi) {                // next sequence with tiles
                ++ib;
                ilo = ihi;
                ihi = P(ib + 1);
                if (ihi > ilo) ilen = L(ib, ilo, ihi);
            }
            const int k0 = (it - ilo) * kTile;
            nkeys = (uint32_t)min(ilen - k0, kTile);
            bytes = nkeys * (uint32_t)kv_row * 2u;
            if constexpr (!Paged) row = ((size_t)ib * a.S_max + k0) * kv_row;
        }
        if constexpr (Paged) {
            if ((issued & (kWindow - 1)) == 0) {
                // lane l: the wave's tile issued + l, i.e. flattened tile it + l * wph
                pw = -1;
                const int tl = it + lane * wph;
                // its sequence: the last b with pre[b] <= tl, by a search whose every step
                // all lanes take (the small-batch table is read across lanes)
                const int tc = min(tl, t1 - 1);
                int bl = 0;
                for (int step = small ? 32 : kMaxDecodeBatch / 2; step > 0; step >>= 1) {
                    const int mid = bl + step;
                    const int pm = P_lane(min(mid, a.B));
                    if (mid < a.B && pm <= tc) bl = mid;
                }
                const int pb = P_lane(bl);
                if (tl < t1) {
                    const int key = (tl - pb) * kTile;
                    const int pg = a.block_table[(size_t)bl * a.max_blocks + key / a.page];
                    if ((unsigned)pg < (unsigned)a.num_pages) {
                        pw = pg * a.page + key % a.page;
                        ppg = pg;
                        prw = key % a.page;
                    }
                }
            }
            const int pr = __builtin_amdgcn_readlane(pw, issued & (kWindow - 1));
            row = (size_t)max(pr, 0) * kv_row;
            if (pr < 0) nkeys = bytes = 0;     // an entry outside the pool reads as zeros
            if constexpr (Fp8) {
                const int pgi = max(__builtin_amdgcn_readlane(ppg, issued & (kWindow - 1)), 0);
                const int rr = __builtin_amdgcn_readlane(prw, issued & (kWindow - 1));
                nkeys = __builtin_amdgcn_readfirstlane(nkeys);
                const uint8_t *pk = reinterpret_cast<const uint8_t *>(a.k) + (size_t)pgi * a.page_bytes;
                const uint8_t *pv = reinterpret_cast<const uint8_t *>(a.v) + (size_t)pgi * a.page_bytes;
                const size_t rowb = (size_t)rr * kv_row + (size_t)hk * D;
                const size_t sc = (size_t)a.page * kv_row + 4u * (size_t)rr;
                load_tile8<D>(r, pk + rowb, pv + rowb, pk + sc, pv + sc, nkeys * (uint32_t)kv_row,
                              nkeys * 4u, toff8, grp);
            }
        }
        bytes = __builtin_amdgcn_readfirstlane(bytes);
        if constexpr (!Fp8) load_tile<D>(r, kbase + row, vbase + row, bytes, toff);
        it += wph;
        ++issued;
    };

    bf16x8 qf[CB][T::KS];
#pragma unroll
    for (int bk = 0; bk < CB; ++bk) load_q<D>(qf[bk], a, cb, hk, G, colb[bk], grp);
    TileRegs<D, Fp8> ring;
    __builtin_amdgcn_sched_barrier(0);
    issue(ring);

    // ---- sweep: one state per sequence the partition touches ----
    int tw = t0 + phase;                       // next tile this wave computes
    while (true) {
        const int slo = P(cb), shend = P(cb + 1);
        const int shi = min(shend, t1);
        const int len = L(cb, slo, shend);
        WaveState<D, CB> st;
        // a column's token sits at position len - 1 - gap and sees keys up to it
        int key_end[CB];
#pragma unroll
        for (int bk = 0; bk < CB; ++bk) {
            st.m[bk] = kNoMax;
            st.l[bk] = 0.f;
            st.lw[bk] = 0.f;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) st.o[bk][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            key_end[bk] = len - gapb[bk];
        }
        for (; tw < shi; tw += wph) {
            f32x4 sc[CB];
            float ksc[4] = {1.f, 1.f, 1.f, 1.f}, vsc[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (Fp8) {
                score_tile8<D, CB>(ring, qf, vs, lane, sc);
                // (whole-vector casts: a bit cast of one vector element reads element 0)
                const f32x4 kf4 = __builtin_bit_cast(f32x4, ring.ksc);
                const f32x4 vf4 = __builtin_bit_cast(f32x4, ring.vsc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ksc[i] = kf4[i];
                    vsc[i] = vf4[i];
                }
            } else {
                score_tile<D, CB>(ring, qf, vs, lane, sc);
            }
            __builtin_amdgcn_sched_barrier(0);
            issue(ring);                       // the next tile's loads go out first
            softmax_pv<D, CB, Fp8>(st, sc, vs, (tw - slo) * kTile, key_end, a.scale_log2, lane,
                                   ksc, vsc);
        }
        finish_state<D, CB>(st);

        // the next sequence with tiles; its Q is requested before this state is stored
        const bool more = shi < t1;
        int nb = cb;
        if (more) {
            ++nb;
            while (P(nb + 1) == P(nb)) ++nb;
#pragma unroll
            for (int bk = 0; bk < CB; ++bk) load_q<D>(qf[bk], a, nb, hk, G, colb[bk], grp);
        }
        const size_t srow = (size_t)(x + cb) * a.H_q * a.T;   // states: [slot][H_q * T]

        if (wph == 1) {
            // one wave per head: its registers hold the whole state.  Lane (row16, grp) holds
            // elements 16 dt + 4 grp .. + 3 of state row row16, so stores from registers would
            // write 32-byte pieces of 8 rows each; the block's rows go through the wave's own
            // V staging area instead (free once its last tile is done; 32-byte segment s of
            // row r at segment s ^ (r mod NDT)) and leave 1 KiB of consecutive rows per store.
            uint8_t *stg = reinterpret_cast<uint8_t *>(vs);
#pragma unroll
            for (int bk = 0; bk < CB; ++bk) {
                const int nh = nhb[bk];
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt)
                    *reinterpret_cast<u32x2 *>(stg + row16 * (2 * D) +
                                               32 * (dt ^ (row16 & (T::NDT - 1))) + 8 * grp) =
                        u32x2{pack_bf16x2(st.o[bk][dt][0], st.o[bk][dt][1]),
                              pack_bf16x2(st.o[bk][dt][2], st.o[bk][dt][3])};
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const size_t row0 = srow + h0 + bk * 16;
                uint8_t *dst = reinterpret_cast<uint8_t *>(a.part_o + row0 * D);
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {   // 16 rows of 2 D bytes, 1 KiB at a time
                    const int byte = i * 1024 + lane * 16;
                    const int r = byte / (2 * D), seg = (byte % (2 * D)) / 32;
                    if (r < nh)
                        *reinterpret_cast<u32x4 *>(dst + byte) = *reinterpret_cast<const u32x4 *>(
                            stg + r * (2 * D) + 32 * (seg ^ (r & (T::NDT - 1))) + byte % 32);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (grp == 0 && row16 < nh) {
                    a.part_m2[row0 + row16] = st.m[bk];
                    a.part_l[row0 + row16] = st.l[bk];
                }
            }
        } else {
            // several waves per head: merge their states through LDS (in the V staging
            // area, which every wave has finished reading), one block of columns at a time:
            // red[w][column][0..D) = O^T column, [D] = m, [D+1] = l
#pragma unroll
            for (int bk = 0; bk < CB; ++bk) {
            const int nh = nhb[bk];
            __syncthreads();
            float *red = reinterpret_cast<float *>(smem);
            constexpr int RS = D + 2;
            float *mine = red + (w * 16 + row16) * RS;
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mine[dt * 16 + grp * 4 + i] = st.o[bk][dt][i];
            if (grp == 0) {
                mine[D] = st.m[bk];
                mine[D + 1] = st.l[bk];
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < a.hpw * nh * D; idx += kWaves * 64) {
                const int hw2 = idx / (nh * D), h = (idx / D) % nh, d = idx % D;
                float M = neg_inf();
                for (int ph = 0; ph < wph; ++ph)
                    M = fmaxf(M, red[((hw2 + a.hpw * ph) * 16 + h) * RS + D]);
                float L = 0.f, O = 0.f;
                for (int ph = 0; ph < wph; ++ph) {
                    const float *rw = red + ((hw2 + a.hpw * ph) * 16 + h) * RS;
                    // a wave with no live key for this column adds nothing
                    const float al = rw[D] == neg_inf() ? 0.f : exp2_fast(rw[D] - M);
                    L += al * rw[D + 1];
                    O += al * rw[d];
                }
                const size_t row = srow + (hgrp * a.hpw + hw2) * GT + hg * CW + bk * 16 + h;
                a.part_o[row * D + d] = __builtin_bit_cast(uint16_t, (__bf16)O);
                if (d == 0) {
                    a.part_m2[row] = L > 0.f ? M : neg_inf();
                    a.part_l[row] = L;
                }
            }
            }
            __syncthreads();   // the staging area is reused by the next sequence
        }
        if (!more) break;
        cb = nb;
    }
}

template <int D, int CB>
hipError_t launch_cb(const DecodeSplitArgs &a, hipStream_t stream) {
    const int GT = a.H_q / a.H_kv * a.T;
    const int n_hg = (GT + 16 * CB - 1) / (16 * CB);
    dim3 grid(a.units, (a.H_kv / a.hpw) * n_hg);
    if (a.fp8) {
        if constexpr (D >= 64)   // (a lane's K codes are at least one 16-byte load)
            hipLaunchKernelGGL((decode_split_kernel<D, true, CB, true>), grid, dim3(kWaves * 64), 0,
                               stream, a, n_hg);
        else
            return hipErrorInvalidValue;
    } else if (a.block_table) {
        hipLaunchKernelGGL((decode_split_kernel<D, true, CB, false>), grid, dim3(kWaves * 64), 0,
                           stream, a, n_hg);
    } else {
        hipLaunchKernelGGL((decode_split_kernel<D, false, CB, false>), grid, dim3(kWaves * 64), 0,
                           stream, a, n_hg);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch(const DecodeSplitArgs &a, hipStream_t stream) {
    return a.cb == 2 ? launch_cb<D, 2>(a, stream) : launch_cb<D, 1>(a, stream);
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
