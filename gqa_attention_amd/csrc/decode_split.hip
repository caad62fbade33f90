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

constexpr int kTile = 32;  // keys per wave iteration = two 16-key MFMA row tiles
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
    u32x4 k[2][DecodeTraits<D>::KS];
    u32x4 v[DecodeTraits<D>::NVI];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &r, const uint16_t *kbase,
                                          const uint16_t *vbase, size_t kv_row, int key0,
                                          int last_key, int lane) {
    using T = DecodeTraits<D>;
    const int row16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        int key = min(key0 + t * 16 + row16, last_key);
        const uint16_t *p = kbase + (size_t)key * kv_row + grp * (D / 4);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) r.k[t][ks] = load16(p + ks * 8);
    }
#pragma unroll
    for (int i = 0; i < T::NVI; ++i) {
        int key = min(key0 + i * T::RPI + lane / T::LPR, last_key);
        r.v[i] = load16(vbase + (size_t)key * kv_row + (lane % T::LPR) * 8);
    }
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

template <int D>
__device__ __forceinline__ void compute_tile(WaveState<D> &st, const TileRegs<D> &r,
                                             const bf16x8 (&qf)[DecodeTraits<D>::KS],
                                             uint16_t *vs, int key0, int key_end,
                                             float scale_log2, int lane) {
    using T = DecodeTraits<D>;
    const int row16 = lane & 15, grp = lane >> 4;

    // S^T = K . Q^T for keys key0..key0+31 (two 16-row tiles)
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) s[t] = mfma16(as_bf16x8(r.k[t][ks]), qf[ks], s[t]);
    }

    // stage the V tile (row-major, padded) for the transposed P.V operand
#pragma unroll
    for (int i = 0; i < T::NVI; ++i) {
        uint16_t *dst = vs + (i * T::RPI + lane / T::LPR) * T::VPITCH + (lane % T::LPR) * 8;
        *reinterpret_cast<u32x4 *>(dst) = r.v[i];
    }

    // scale to log2 units; keys past the slab/sequence end are masked
    float s2[8];
    float mx = neg_inf();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int key = key0 + t * 16 + grp * 4 + i;
            float x = key < key_end ? s[t][i] * scale_log2 : neg_inf();
            s2[t * 4 + i] = x;
            mx = fmaxf(mx, x);
        }
    // Each lane holds 8 of a head's 32 scores.  Only when one of them passes the shared
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

    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = exp2_fast(s2[j] - st.m);
        st.l += p[j];
    }
    // P^T as the B operand: slot j of lane group grp is key (j/4)*16 + 4*grp + j%4
    const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.lw = add_bf16_pair(pw[i], st.lw);

    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T.  V^T fragment of lane (row16, grp): column d = 16*dt + row16,
    // keys 4*grp + 0..3 and 16 + 4*grp + 0..3, via two LDS transpose reads whose lanes
    // point at row 4*grp + row16/4, columns 16*dt + 4*(row16%4).
    const uint16_t *vrow = vs + (4 * grp + (row16 >> 2)) * T::VPITCH + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) {
        const u32x2 lo = lds_read_tr16(vrow + dt * 16);
        const u32x2 hi = lds_read_tr16(vrow + 16 * T::VPITCH + dt * 16);
        const bf16x8 vf = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        st.o[dt] = mfma16(vf, pf, st.o[dt]);
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

template <int D>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(DecodeSplitArgs a, int n_hg) {
    using T = DecodeTraits<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * kTile * T::VPITCH];

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

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row16 = lane & 15, grp = lane >> 4;
    // wave w sweeps KV head hw of this workgroup's group; the wph waves of one head take
    // interleaved 32-key tiles of the slab (phase = first tile)
    const int wph = kWaves / a.hpw;
    const int hw = w % a.hpw, phase = w / a.hpw;
    const int hk = hgrp * a.hpw + hw;
    const int h0 = hk * G + hg * 16;
    const int nh = min(16, G - hg * 16);
    const size_t n_states = (size_t)a.P * a.slabs;
    const size_t state0 = ((size_t)b * a.H_q + h0) * n_states + (size_t)p * a.slabs + sl;

    if (s0 >= s1) {  // a slab past the end of a live chunk: mark its states empty
        if (phase == 0 && lane < nh) {
            a.part_m2[state0 + lane * n_states] = neg_inf();
            a.part_l[state0 + lane * n_states] = 0.f;
        }
        return;
    }

    // Q^T fragments (B operand): column = query head h0 + row16, k-slots = d
    bf16x8 qf[T::KS];
    {
        const uint16_t *qrow =
            a.q + ((size_t)b * a.H_q + h0 + min(row16, nh - 1)) * D + grp * (D / 4);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            u32x4 x = load16(qrow + ks * 8);
            if (row16 >= nh) x = u32x4{0u, 0u, 0u, 0u};
            qf[ks] = as_bf16x8(x);
        }
    }

    const size_t kv_row = (size_t)a.H_kv * D;
    const size_t head_off = ((size_t)b * a.S_max * a.H_kv + hk) * D;
    const uint16_t *kbase = a.k + head_off;
    const uint16_t *vbase = a.v + head_off;
    uint16_t *vs = smem + w * kTile * T::VPITCH;

    WaveState<D> st;
    st.m = neg_inf();
    st.l = 0.f;
    st.lw = 0.f;
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This wave's tiles are phase, phase + wph, ...; tile i starts at key0(i).  The loop is
    // written so that every compute is preceded, on its own path, by an unconditional
    // prefetch of the next tile (or by nothing, for the last tile): the load counter then
    // only has to drain the current tile's loads, never the prefetch.
    const int ntiles = (s1 - s0 + kTile - 1) / kTile;
    const int n_w = phase < ntiles ? (ntiles - 1 - phase) / wph + 1 : 0;
    const int last_key = s1 - 1;
    auto key0 = [&](int i) { return s0 + (phase + i * wph) * kTile; };
    TileRegs<D> ra, rb;
    if (n_w > 0) {
        load_tile<D>(ra, kbase, vbase, kv_row, key0(0), last_key, lane);
        for (int i = 0;; i += 2) {
            if (i + 1 >= n_w) {
                compute_tile<D>(st, ra, qf, vs, key0(i), s1, a.scale_log2, lane);
                break;
            }
            load_tile<D>(rb, kbase, vbase, kv_row, key0(i + 1), last_key, lane);
            compute_tile<D>(st, ra, qf, vs, key0(i), s1, a.scale_log2, lane);
            if (i + 2 >= n_w) {
                compute_tile<D>(st, rb, qf, vs, key0(i + 1), s1, a.scale_log2, lane);
                break;
            }
            load_tile<D>(ra, kbase, vbase, kv_row, key0(i + 2), last_key, lane);
            compute_tile<D>(st, rb, qf, vs, key0(i + 1), s1, a.scale_log2, lane);
        }
    }

    finish_state<D>(st);

    if (wph == 1) {
        // one wave per head: its registers hold the slab's whole state
        if (row16 < nh) {
            const size_t row = state0 + row16 * n_states;
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
        const size_t row = ((size_t)b * a.H_q + hk2 * G + hg * 16 + h) * n_states +
                           (size_t)p * a.slabs + sl;
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
    hipLaunchKernelGGL(decode_split_kernel<D>, grid, dim3(kWaves * 64), 0, stream, a, n_hg);
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
