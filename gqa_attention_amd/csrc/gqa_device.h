// gqa_device.h -- device-side types and helpers shared by the gfx950 kernels.
//
// Vector types follow the operand shapes of the CDNA4 bf16 matrix-core
// instructions used here:
//   v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, C/D 16x16 fp32.  Each lane holds
//     8 bf16 of A (row lane%16, k-slots 8*(lane/16)..+7), 8 bf16 of B (column
//     lane%16, the same k-slots) and 4 fp32 of D (rows 4*(lane/16)..+3, column
//     lane%16).
//   v_mfma_f32_32x32x16_bf16: A 32x16, B 16x32, C/D 32x32 fp32.  Each lane holds
//     8 bf16 of A (row lane%32, k-slots 8*(lane/32)..+7), 8 of B (column
//     lane%32, same k-slots) and 16 fp32 of D (rows 8*(r/4) + 4*(lane/32) + r%4
//     for r = 0..15, column lane%32).
// Since A and B use the same lane/slot -> k assignment, any permutation of the
// reduction index that is applied to both operands leaves the product
// unchanged; the kernels use that freedom to make every lane's slots
// contiguous in memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Buffer resource over [base, base + bytes) for raw (unstrided) buffer loads: a load at a
// byte offset >= bytes returns zeros and touches no memory.  Word 3 is the gfx9-family
// default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes at byte offset voff + imm of a buffer (imm a compile-time constant < 4096).
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int imm) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff + imm, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> two bf16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// acc + lo + hi of a packed bf16 pair, in fp32 (v_dot2 against (1, 1)).  The kernels
// sum the softmax denominator from the same bf16-rounded P that enters the P.V matrix
// product, so the output is an exact convex combination of the weights actually used.
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives 16-bit element (i % 4) of the 8-byte chunks addressed by lanes
// 4e + i/4, e = 0..3 (layout checked on the device).  So if lane j of a group
// points at row k0 + j/4, columns n0 + 4*(j%4) of a row-major 16-bit tile, lane i
// receives rows k0..k0+3 of column n0 + i: four consecutive reduction-index values
// of one output column, as a matrix-core operand wants them.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Store the 32 rows of a wave's four 32x32 accumulator tiles x (d = 128; times f, rounded
// to bf16) to rows r0 .. r0 + 31 of out (row_elems elements apart; rows at or past n_rows are
// not stored).  A lane holds elements 32 dt + 8 rq + 4 hf .. + 3 of row r0 + lane % 32, so
// stores from registers would touch 32 rows per instruction; the rows go through the wave's
// own 8 KiB of LDS (stage; 16-byte chunks XOR-permuted by row, which keeps the 16-byte reads
// free of bank conflicts) and leave as whole 256-byte rows.
__device__ __forceinline__ void store_rows128(const f32x16 (&x)[4], float f, uint8_t *stage,
                                              uint16_t *out, size_t row_elems, int r0,
                                              int n_rows, int lane) {
    const int r32 = lane & 31, hf = lane >> 5, cr = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int r = rq * 4;
            const int c = (dt * 4 + rq) ^ (r32 & 15);
            *reinterpret_cast<u32x2 *>(stage + r32 * 256 + 16 * c + 8 * hf) =
                u32x2{pack_bf16x2(x[dt][r] * f, x[dt][r + 1] * f),
                      pack_bf16x2(x[dt][r + 2] * f, x[dt][r + 3] * f)};
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const u32x4 val =
            *reinterpret_cast<const u32x4 *>(stage + rr * 256 + 16 * (cr ^ (rr & 15)));
        if (r0 + rr < n_rows)
            *reinterpret_cast<u32x4 *>(out + (size_t)(r0 + rr) * row_elems + 8 * cr) = val;
    }
}

}  // namespace gqa
