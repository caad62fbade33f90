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
// One wavefront per (b, h): lanes share the partial loop for M and L with a
// butterfly reduction, then each lane accumulates D/64 output columns.  The
// merge order is fixed, so results are run-to-run deterministic.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

__device__ __forceinline__ float wave_reduce_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_reduce_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

template <int D>
__global__ __launch_bounds__(64) void lse_merge_kernel(MergeArgs a) {
    constexpr int EPL = (D + 63) / 64;  // output columns per lane
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;

    int n = a.P;
    if (a.counts) {
        int c = a.counts[b];
        if (a.counts_are_lengths) {
            c = min(max(c, 0), a.S_max);
            n = (c + a.chunk - 1) / a.chunk;
        } else {
            n = min(max(c, 0), a.P);
        }
    }
    const size_t row = (size_t)b * a.H_q + h;
    const float *m2 = a.part_m2 + row * a.P;
    const float *lp = a.part_l + row * a.P;
    const float *op = a.part_o + row * a.P * D;

    float M = neg_inf();
    for (int p = lane; p < n; p += 64) M = fmaxf(M, m2[p]);
    M = wave_reduce_max(M);

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float L = 0.f;
    if (M != neg_inf()) {
        for (int p = lane; p < n; p += 64) L += exp2_fast(m2[p] - M) * lp[p];
        L = wave_reduce_sum(L);
#pragma unroll 8
        for (int p = 0; p < n; ++p) {
            const float al = exp2_fast(m2[p] - M);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int d = lane + 64 * e;
                if (d < D) acc[e] += al * op[(size_t)p * D + d];
            }
        }
    }
    const bool empty = (M == neg_inf());
    const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int d = lane + 64 * e;
        if (d < D) {
            const uint32_t packed = pack_bf16x2(acc[e] * inv, 0.f);
            a.o[row * D + d] = (uint16_t)(packed & 0xFFFFu);
        }
    }
    if (lane == 0) a.lse[row] = empty ? neg_inf() : kLn2 * (M + __builtin_log2f(L));
}

template <int D>
hipError_t launch(const MergeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(lse_merge_kernel<D>, dim3(a.H_q, a.B), dim3(64), 0, stream, a);
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
