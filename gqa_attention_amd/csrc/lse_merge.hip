// lse_merge.hip -- stage 2 of split-KV decode on gfx950: merge partial states.
//
// For each (sequence b, query head h), over its partials p < n_b
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
// Sixteen waves per (b, h): wave w folds the partials p = w, w+16, ... into a running
// (M, L, O) with the same online update, in batches whose loads are all issued before
// any is used (one memory round trip per 256 partials of a row), then the sixteen wave
// states are merged through LDS.  The order is fixed, so results are run-to-run
// deterministic.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kMergeWaves = 16;
constexpr int kBatch = 16;     // partials per wave per memory round trip

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void lse_merge_kernel(MergeArgs a) {
    constexpr int EPL = (D + 63) / 64;  // output columns per lane
    __shared__ float red[kMergeWaves][D + 2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    int n = a.P;
    if (a.counts) {
        int c = a.counts[b];
        if (a.counts_are_lengths) {
            c = min(max(c, 0), a.S_max);
            n = (c + a.chunk - 1) / a.chunk * a.slabs;
        } else {
            n = min(max(c, 0), a.P);
        }
    }
    const size_t row = (size_t)b * a.H_q + h;
    const float *m2 = a.part_m2 + row * a.P;
    const float *lp = a.part_l + row * a.P;
    const float *op = a.part_o + row * a.P * D;

    // running state of this wave (uniform M and L; O spread over lanes)
    float M = neg_inf(), L = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    // Batches of kBatch partials: all loads of a batch are issued (clamped indices,
    // unconditional) before any is used, so one memory round trip serves the batch.
    for (int base = w; base < n; base += kMergeWaves * kBatch) {
        float mv[kBatch], lv[kBatch], ov[kBatch][EPL];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = min(base + j * kMergeWaves, n - 1);
            mv[j] = m2[p];
            lv[j] = lp[p];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int d = lane + 64 * e;
                ov[j][e] = d < D ? op[(size_t)p * D + d] : 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const float mp = mv[j];
            // past the end, or an empty partial: the state is unchanged
            const bool use = (base + j * kMergeWaves < n) && (mp != neg_inf());
            const float m_new = fmaxf(M, mp);
            const float a_old = exp2_fast(M - m_new);  // 2^-inf = 0 while the state is empty
            const float a_p = exp2_fast(mp - m_new);
            L = use ? L * a_old + a_p * lv[j] : L;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = use ? acc[e] * a_old + a_p * ov[j][e] : acc[e];
            M = use ? m_new : M;
        }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int d = lane + 64 * e;
        if (d < D) red[w][d] = acc[e];
    }
    if (lane == 0) {
        red[w][D] = M;
        red[w][D + 1] = L;
    }
    __syncthreads();
    if (w != 0) return;

    float Mt = neg_inf();
#pragma unroll
    for (int ww = 0; ww < kMergeWaves; ++ww) Mt = fmaxf(Mt, red[ww][D]);
    const bool empty = (Mt == neg_inf());
    float al[kMergeWaves], Lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < kMergeWaves; ++ww) {
        al[ww] = empty ? 0.f : exp2_fast(red[ww][D] - Mt);
        Lt += al[ww] * red[ww][D + 1];
    }
    const float inv = empty ? 0.f : 1.f / Lt;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int d = lane + 64 * e;
        if (d < D) {
            float o = 0.f;
#pragma unroll
            for (int ww = 0; ww < kMergeWaves; ++ww) o += al[ww] * red[ww][d];
            a.o[row * D + d] = (uint16_t)(pack_bf16x2(o * inv, 0.f) & 0xFFFFu);
        }
    }
    if (lane == 0) a.lse[row] = empty ? neg_inf() : kLn2 * (Mt + __builtin_log2f(Lt));
}

template <int D>
hipError_t launch(const MergeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(lse_merge_kernel<D>, dim3(a.H_q, a.B), dim3(kMergeWaves * 64), 0, stream, a);
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
