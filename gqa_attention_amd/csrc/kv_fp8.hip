// kv_fp8.hip -- FP8 (E4M3) paged KV cache: per-token quantisation into pages on gfx950.
//
// The cache format of "Attention Kernel lineage" (V07), section 17.7: every page of a pool
// holds its `page` token rows of E4M3 codes ([page][H_kv][d] bytes), followed by the page's
// `page` per-token fp32 scales (the B_p scalars appended to the page); the decode kernel
// dequantises as it loads.  A token's row of one pool (its H_kv * d values) shares one
// scale 2^e, e the smallest integer with max |x| <= 448 * 2^e (448: the largest finite
// E4M3 value), clamped to [-126, 127] (an all-zero row takes -126).  A power of two makes
// x * 2^-e exact, so each code is the E4M3 value nearest to x * 2^-e (ties to even), as
// v_cvt_pk_fp8_f32 rounds, and code * 2^e is exactly a bfloat16.
//
// One wave quantises one token row: a pass for max |x|, a wave reduction, then the codes.
// This writes the cache (the step upstream of attention); the attention kernels only read.
// The inverse (kv_dequantize_fp8) writes a pool's live tokens back as a bf16 cache, so that
// kernels reading bf16 -- the chunked prefill -- can run on an FP8 cache.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int kWavesPerBlock = 4;

// The scale exponent of a row whose largest magnitude is amax (>= 0, finite).  With
// amax = m 2^E, m in [0.5, 1): 448 * 2^(E-9) = 1.75 * 2^(E-1) is the first candidate, else
// E - 8; every comparison is exact in fp32.
__device__ __forceinline__ int scale_exponent(float amax) {
    // (below 2^-126 the answer is the clamp, whatever the denormal mode)
    if (!(amax >= 0x1p-126f)) return -126;
    const int E = __builtin_amdgcn_frexp_expf(amax);
    int e = E - 9;
    if (amax > __builtin_amdgcn_ldexpf(448.f, e)) ++e;
    return max(min(e, 127), -126);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__global__ __launch_bounds__(kWavesPerBlock * 64) void kv_quantize_fp8_kernel(KvQuantArgs a) {
    const int lane = threadIdx.x & 63;
    const long tok = (long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (tok >= (long)a.B * a.S_max) return;          // (whole waves)
    const int b = (int)(tok / a.S_max), t = (int)(tok % a.S_max);
    const int len = a.seqlens ? min(max(a.seqlens[b], 0), a.S_max) : a.S_max;
    if (t >= len) return;
    const int pg = a.block_table[(size_t)b * a.max_blocks + t / a.page];
    if (pg < 0 || pg >= a.num_pages) return;          // a slot outside the pool is not written
    const int W = a.H_kv * a.d;                       // values per token row (a multiple of 8)
    const uint16_t *row = a.x + ((size_t)b * a.S_max + t) * W;

    float amax = 0.f;
    for (int c = lane * 8; c < W; c += 512) {
        const u32x4 v = load16(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const int e = scale_exponent(amax);

    uint8_t *page_base = a.pool + (size_t)pg * a.page_bytes;
    uint8_t *dst = page_base + (size_t)(t % a.page) * W;
    for (int c = lane * 8; c < W; c += 512) {
        const u32x4 v = load16(row + c);
        u32x2 codes;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int w = 0;
            w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(bf16_lo(v[2 * h]), -e),
                                                __builtin_amdgcn_ldexpf(bf16_hi(v[2 * h]), -e), w,
                                                false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(bf16_lo(v[2 * h + 1]), -e),
                                                __builtin_amdgcn_ldexpf(bf16_hi(v[2 * h + 1]), -e),
                                                w, true);
            codes[h] = (uint32_t)w;
        }
        *reinterpret_cast<u32x2 *>(dst + c) = codes;
    }
    if (lane == 0)
        *reinterpret_cast<float *>(page_base + (size_t)a.page * W + 4 * (t % a.page)) =
            __builtin_amdgcn_ldexpf(1.f, e);
}

// The inverse, one wave per token row: eight codes at a time become bf16 (exactly: every
// E4M3 value is a bfloat16), are multiplied by the row's power-of-two scale in fp32 (exact)
// and written as bf16 (exact again, so the row is the dequantised cache the decode reads).
__global__ __launch_bounds__(kWavesPerBlock * 64) void kv_dequantize_fp8_kernel(KvDequantArgs a) {
    const int lane = threadIdx.x & 63;
    const long tok = (long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (tok >= (long)a.B * a.S_max) return;          // (whole waves)
    const int b = (int)(tok / a.S_max), t = (int)(tok % a.S_max);
    const int len = a.seqlens ? min(max(a.seqlens[b], 0), a.S_max) : a.S_max;
    if (t >= len) return;
    const int pg = a.block_table[(size_t)b * a.max_blocks + t / a.page];
    const int W = a.H_kv * a.d;                       // values per token row (a multiple of 8)
    uint16_t *row = a.x + ((size_t)b * a.S_max + t) * W;
    if (pg < 0 || pg >= a.num_pages) {                // a page outside the pool reads as zeros
        for (int c = lane * 8; c < W; c += 512) *reinterpret_cast<u32x4 *>(row + c) = u32x4{0, 0, 0, 0};
        return;
    }
    const uint8_t *page_base = a.pool + (size_t)pg * a.page_bytes;
    const uint8_t *src = page_base + (size_t)(t % a.page) * W;
    const float s = *reinterpret_cast<const float *>(page_base + (size_t)a.page * W + 4 * (t % a.page));
    for (int c = lane * 8; c < W; c += 512) {
        const u32x2 codes = *reinterpret_cast<const u32x2 *>(src + c);
        u32x4 out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes[h], 1.f, false);
            const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)codes[h], 1.f, true);
            const uint32_t wl = __builtin_bit_cast(uint32_t, lo), wh = __builtin_bit_cast(uint32_t, hi);
            out[2 * h] = pack_bf16x2(bf16_lo(wl) * s, bf16_hi(wl) * s);
            out[2 * h + 1] = pack_bf16x2(bf16_lo(wh) * s, bf16_hi(wh) * s);
        }
        *reinterpret_cast<u32x4 *>(row + c) = out;
    }
}

}  // namespace

hipError_t launch_kv_dequantize_fp8(const KvDequantArgs &a, hipStream_t stream) {
    const long toks = (long)a.B * a.S_max;
    hipLaunchKernelGGL(kv_dequantize_fp8_kernel,
                       dim3((unsigned)((toks + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kWavesPerBlock * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_quantize_fp8(const KvQuantArgs &a, hipStream_t stream) {
    const long toks = (long)a.B * a.S_max;
    hipLaunchKernelGGL(kv_quantize_fp8_kernel,
                       dim3((unsigned)((toks + kWavesPerBlock - 1) / kWavesPerBlock)),
                       dim3(kWavesPerBlock * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gqa
