// mfma_rate.hip -- the prefill's matrix-core ceiling for a given operand distribution.
//
// The causal prefill is bound by its bf16 matrix products (V07 section 19: prefill is
// compute-bound).  How fast the matrix cores run those products on one device depends on
// the operand bits as well as on the instruction stream: under sustained load the chip
// lowers its engine clock with the switching activity of the multiplier arrays, so random
// mantissas (the prefill's Q, K, V and P) run measurably slower than zeros or constants.
// This kernel measures that rate: every wave of one 512-thread workgroup per compute unit
// runs rounds of 16 independent v_mfma_f32_32x32x16_bf16 products (four accumulators, no
// dependent chain), on 16 operand fragments it loads once from the caller's buffer, and
// nothing else.  The caller times it and divides the FLOP count by the time.
//
// Each thread stores the sum of its accumulators to the sink, so the products stay.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kRateThreads = 512;
constexpr int kRateBlocks = 256;
constexpr int kRatePadBytes = 96 * 1024;   // LDS held so that a compute unit takes one workgroup

__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(const u32x4 *__restrict__ ops,
                                                                 size_t n16, int iters,
                                                                 float *sink) {
    __shared__ uint8_t pad[kRatePadBytes];
    const size_t tid = (size_t)blockIdx.x * kRateThreads + threadIdx.x;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = as_bf16x8(ops[(tid * 16 + 2 * i) % n16]);
        b[i] = as_bf16x8(ops[(tid * 16 + 2 * i + 1) % n16]);
    }
    // (never true for a launch that has threads: keeps the LDS allocation)
    if (iters < 0) pad[threadIdx.x] = 1;
    f32x16 o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = mfma32(a[(2 * j + d) & 7], b[(j + 3 * d) & 7], o[d]);
    }
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += o[d][r];
    sink[tid] = acc;
}

}  // namespace

int mfma_rate_threads() { return kRateThreads * kRateBlocks; }

double mfma_rate_flop(int iters) {
    return (double)kRateBlocks * (kRateThreads / 64) * iters * 16 * (2.0 * 32 * 32 * 16);
}

hipError_t launch_mfma_rate(const void *ops, size_t bytes, int iters, float *sink,
                            hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(kRateBlocks), dim3(kRateThreads), 0, stream,
                       static_cast<const u32x4 *>(ops), bytes / 16, iters, sink);
    return hipGetLastError();
}

}  // namespace gqa
