// lse_merge.hip -- stage 2 of split-KV decode on gfx950: merge partial states.
//
// For each (sequence b, query row: head h and, for a multi-token decode, token i),
// over its partials p < n_b
// ("Attention Kernel lineage" (V07), section 3 merge formula and section 17,
// second stage of split-K decode; ADR-0060 "AHBM GQA Fused Attention",
// section 4, merge of (m, l, O) triplets):
//   M = max_p m2_p,  a_p = 2^(m2_p - M),  L = sum_p a_p l_p,
//   O = (sum_p a_p O_p) / L  -> bf16,     LSE = ln2 * (M + log2 L).
// Partial maxima are in log2 units, so the exponentials are exp2 and the LSE
// is converted back to natural-log units at the end.  A partial with
// m2 = -inf is empty (a_p = 0); a row with no non-empty partial gets O = 0 and
// LSE = -inf (the identity state of the merge, V07 section 3).
//
// The decode's own states hold O in bf16 (m2 and l in fp32); caller-provided partials are
// fp32 throughout.  When every sequence of the decode has the same length, the merge finds
// a sequence's states from the split plan itself instead of reading the split kernel's
// slot table (one dependent memory round trip less).
//
// A row's columns are cut into 32-wide slices, one workgroup of 4 waves per (row, slice),
// so a row's partials are read by D/32 compute units at once.  Each workgroup folds every
// partial's (m2, l) (the few bytes every slice needs) and its slice of O.  Lane l of a wave
// takes columns 4*(l%8) .. +3 of the slice and the partials p = 64*w + 8*j + l/8 (+ 256 per
// round), j < 8: eight 16-byte loads a lane, all in flight together, and only for partials
// that exist.  The lane states are then merged across the 8 lanes of a column group (three
// cross-lane steps) and across the 4 waves through LDS.  The order is fixed, so results are
// run-to-run deterministic.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kMergeWaves = 4;
constexpr int kSlice = 32;                 // columns per workgroup
constexpr int kPerRound = kMergeWaves * 64;  // partials per round (8 per lane)

struct MState {
    float m, l, o[4];
};

// Merge state y into x (either may be empty: m = -inf).
__device__ __forceinline__ void merge_into(MState &x, const MState &y) {
    const float mn = fmaxf(x.m, y.m);
    const float ax = x.m == neg_inf() ? 0.f : exp2_fast(x.m - mn);
    const float ay = y.m == neg_inf() ? 0.f : exp2_fast(y.m - mn);
    x.l = ax * x.l + ay * y.l;
#pragma unroll
    for (int e = 0; e < 4; ++e) x.o[e] = ax * x.o[e] + ay * y.o[e];
    x.m = mn;
}

// Four consecutive O values of a partial state as loaded: fp32, or bf16 (the decode
// workspace: two words of two values each, widened by o4_value after every load of a round
// has been issued -- widening inside the load's own branch would make each load wait).
template <bool OB>
struct ORaw {
    f32x4 v;
};
template <>
struct ORaw<true> {
    u32x2 v;
};

template <bool OB>
__device__ __forceinline__ ORaw<OB> load_o4(const void *base, size_t idx) {
    if constexpr (OB)
        return {*reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(base) + idx)};
    else
        return {*reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx)};
}

template <bool OB>
__device__ __forceinline__ ORaw<OB> zero_o4() {
    if constexpr (OB)
        return {u32x2{0u, 0u}};
    else
        return {f32x4{0.f, 0.f, 0.f, 0.f}};
}

template <bool OB>
__device__ __forceinline__ f32x4 o4_value(const ORaw<OB> &r) {
    if constexpr (OB) {
        const u32x2 w = r.v;
        return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xFFFF0000u),
                     __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xFFFF0000u)};
    } else {
        return r.v;
    }
}

template <int D, bool OB>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_kernel(MergeArgs a) {
    constexpr int NS = D / kSlice;
    __shared__ float red[kMergeWaves][8][6];
    const int r = blockIdx.x / NS, q = blockIdx.x % NS, b = blockIdx.y;   // row r = h * T + i
    const int h = r / a.T, i = r % a.T;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 7, s8 = lane >> 3;

    int n;
    size_t row0;
    if (a.uniform_tiles > 0) {
        // the split plan restated: tile t of the B * uniform_tiles went to partition
        // floor(t * W / tot), and partition x holds its state of sequence b in slot x + b
        const long tot = (long)a.B * a.uniform_tiles;
        const long W = min((long)a.units, tot);
        const long lo = (long)b * a.uniform_tiles, hi = lo + a.uniform_tiles;
        const long x0 = lo * W / tot, x1 = (hi - 1) * W / tot;
        n = (int)(x1 - x0 + 1);
        row0 = (size_t)(x0 + b) * a.state_stride + (size_t)r * a.head_stride;
    } else if (a.seg) {
        n = a.seg[2 * b + 1];
        row0 = (size_t)a.seg[2 * b] * a.state_stride + (size_t)r * a.head_stride;
    } else {
        n = a.counts ? min(max(a.counts[b], 0), a.P) : a.P;
        row0 = (size_t)b * a.batch_stride + (size_t)r * a.head_stride;
    }
    const size_t ss = a.state_stride;
    const float *m2 = a.part_m2 + row0;
    const float *lp = a.part_l + row0;
    const size_t oi = row0 * D + q * kSlice + 4 * c;   // element index of partial 0

    MState st{neg_inf(), 0.f, {0.f, 0.f, 0.f, 0.f}};
    for (int base = 64 * w; base < n; base += kPerRound) {
        float mv[8], lv[8];
        ORaw<OB> ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int p = base + 8 * j + s8;
            if (p < n) {
                mv[j] = m2[p * ss];
                lv[j] = lp[p * ss];
                ov[j] = load_o4<OB>(a.part_o, oi + (size_t)p * ss * D);
            } else {
                mv[j] = neg_inf();
                lv[j] = 0.f;
                ov[j] = zero_o4<OB>();
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // past the end, or an empty partial: m = -inf adds nothing
            const f32x4 o4 = o4_value<OB>(ov[j]);
            const MState y{mv[j], lv[j], {o4[0], o4[1], o4[2], o4[3]}};
            merge_into(st, y);
        }
    }
    // the 8 lanes of a column group (lane bits 3..5)
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
        MState y;
        y.m = __shfl_xor(st.m, off);
        y.l = __shfl_xor(st.l, off);
#pragma unroll
        for (int e = 0; e < 4; ++e) y.o[e] = __shfl_xor(st.o[e], off);
        merge_into(st, y);
    }
    if (lane < 8) {
        red[w][c][0] = st.m;
        red[w][c][1] = st.l;
#pragma unroll
        for (int e = 0; e < 4; ++e) red[w][c][2 + e] = st.o[e];
    }
    __syncthreads();
    if (threadIdx.x >= 8) return;
    MState t{red[0][c][0], red[0][c][1], {red[0][c][2], red[0][c][3], red[0][c][4], red[0][c][5]}};
#pragma unroll
    for (int v = 1; v < kMergeWaves; ++v) {
        const MState y{red[v][c][0], red[v][c][1],
                       {red[v][c][2], red[v][c][3], red[v][c][4], red[v][c][5]}};
        merge_into(t, y);
    }
    const bool empty = t.m == neg_inf();
    const float inv = empty ? 0.f : 1.f / t.l;
    const u32x2 packed = {pack_bf16x2(t.o[0] * inv, t.o[1] * inv),
                          pack_bf16x2(t.o[2] * inv, t.o[3] * inv)};
    *reinterpret_cast<u32x2 *>(a.o + (((size_t)b * a.T + i) * a.H_q + h) * D + q * kSlice + 4 * c) =
        packed;
    if (q == 0 && c == 0)
        a.lse[((size_t)b * a.H_q + h) * a.T + i] =
            empty ? neg_inf() : kLn2 * (t.m + __builtin_log2f(t.l));
}

template <int D>
hipError_t launch(const MergeArgs &a, hipStream_t stream) {
    const dim3 grid(a.H_q * a.T * (D / kSlice), a.B);
    if (a.o_bf16)
        hipLaunchKernelGGL((lse_merge_kernel<D, true>), grid, dim3(kMergeWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((lse_merge_kernel<D, false>), grid, dim3(kMergeWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs &a, hipStream_t stream) {
    switch (a.d) {
    case 32: return launch<32>(a, stream);
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gqa
