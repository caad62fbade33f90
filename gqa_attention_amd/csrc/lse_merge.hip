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
// Sixteen waves per (b, h), split into 32 half-waves: half-wave i folds the partials
// p = i, i+32, ... into a running (M, L, O) with the same online update, its 32 lanes
// each holding D/32 consecutive columns (16-byte loads at d = 128).  A batch's loads are
// all issued before any is used, so one memory round trip serves 256 partials of a row.
// The 32 half-wave states are then merged through LDS, one output column per thread.
// The order is fixed, so results are run-to-run deterministic.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kMergeWaves = 16;
constexpr int kHalves = 2 * kMergeWaves;
constexpr int kBatch = 8;      // partials per half-wave per memory round trip

template <int N>
struct FloatVec {
    float v[N];
};

template <int N>
__device__ __forceinline__ FloatVec<N> load_floats(const float *p) {
    FloatVec<N> r;
    if constexpr (N == 4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = x[i];
    } else if constexpr (N == 2) {
        const f32x2 x = *reinterpret_cast<const f32x2 *>(p);
        r.v[0] = x[0];
        r.v[1] = x[1];
    } else {
        r.v[0] = *p;
    }
    return r;
}

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_kernel(MergeArgs a) {
    constexpr int DPL = D / 32;           // columns per lane of a half-wave
    __shared__ float red[kHalves][D + 2];
    const int r = blockIdx.x, b = blockIdx.y;     // row r = h * T + i
    const int h = r / a.T, i = r % a.T;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = 2 * w + (lane >> 5), hl = lane & 31;

    int n;
    size_t row0;
    if (a.seg) {
        n = a.seg[2 * b + 1];
        row0 = (size_t)a.seg[2 * b] * a.state_stride + (size_t)r * a.head_stride;
    } else {
        n = a.counts ? min(max(a.counts[b], 0), a.P) : a.P;
        row0 = (size_t)b * a.batch_stride + (size_t)r * a.head_stride;
    }
    const size_t ss = a.state_stride;
    const float *m2 = a.part_m2 + row0;
    const float *lp = a.part_l + row0;
    const float *op = a.part_o + row0 * D + hl * DPL;

    float M = neg_inf(), L = 0.f;
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
    for (int base = half; base < n; base += kHalves * kBatch) {
        float mv[kBatch], lv[kBatch];
        FloatVec<DPL> ov[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = min(base + j * kHalves, n - 1);   // clamped: loads stay in range
            mv[j] = m2[p * ss];
            lv[j] = lp[p * ss];
            ov[j] = load_floats<DPL>(op + (size_t)p * ss * D);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const float mp = mv[j];
            // past the end, or an empty partial: the state is unchanged
            const bool use = (base + j * kHalves < n) && (mp != neg_inf());
            const float m_new = fmaxf(M, mp);
            const float a_old = exp2_fast(M - m_new);  // 2^-inf = 0 while the state is empty
            const float a_p = exp2_fast(mp - m_new);
            L = use ? L * a_old + a_p * lv[j] : L;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = use ? acc[e] * a_old + a_p * ov[j].v[e] : acc[e];
            M = use ? m_new : M;
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) red[half][hl * DPL + e] = acc[e];
    if (hl == 0) {
        red[half][D] = M;
        red[half][D + 1] = L;
    }
    __syncthreads();

    // combine the 32 half-wave states: one output column per thread
    if (threadIdx.x >= D) return;
    const int d = threadIdx.x;
    float Mt = neg_inf();
#pragma unroll
    for (int i = 0; i < kHalves; ++i) Mt = fmaxf(Mt, red[i][D]);
    const bool empty = (Mt == neg_inf());
    float Lt = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < kHalves; ++i) {
        const float al = empty ? 0.f : exp2_fast(red[i][D] - Mt);
        Lt += al * red[i][D + 1];
        o += al * red[i][d];
    }
    const float inv = empty ? 0.f : 1.f / Lt;
    a.o[(((size_t)b * a.T + i) * a.H_q + h) * D + d] = (uint16_t)(pack_bf16x2(o * inv, 0.f) & 0xFFFFu);
    if (d == 0)
        a.lse[((size_t)b * a.H_q + h) * a.T + i] =
            empty ? neg_inf() : kLn2 * (Mt + __builtin_log2f(Lt));
}

template <int D>
hipError_t launch(const MergeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(lse_merge_kernel<D>, dim3(a.H_q * a.T, a.B), dim3(kMergeWaves * 64), 0,
                       stream, a);
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
