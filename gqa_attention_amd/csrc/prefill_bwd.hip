// prefill_bwd.hip -- backward of whole-prompt causal GQA prefill on gfx950.
//
// Given the forward's O and LSE and the output gradient dO, the input gradients are
// ("Attention Kernel lineage" (V07), section 6.1):
//   P_ij = exp(s_ij - LSE_i)    dP_ij = dO_i . v_j    D_i = sum_j P_ij dP_ij = dO_i . O_i
//   dS_ij = P_ij (dP_ij - D_i)  dQ_i = tau sum_j dS_ij k_j
//   dK_j = tau sum_i dS_ij q_i  dV_j = sum_i P_ij dO_i      (causal pairs j <= i)
// and a KV head's dK and dV add up the contributions of its G query heads (section 14).
// P is never stored: each kernel forms it again from the row's LSE (section 6.3, recompute).
//
// Three launches:
//   bwd_prep   D_i as the row-wise dot of O and dO (section 6.2) and LSE in log2 units, kept
//              per 64-row block as [lse2 x 64 | D x 64] so one DMA fetches a block's pair;
//   bwd_dq     query-block outer, key tiles inner, dQ accumulated in registers: no atomics
//              (section 8: Q outer removes the dQ atomics of the section 6.4 loop);
//   bwd_dkdv   key-block outer, query tiles inner (the loop of section 6.4 without its dQ
//              update), one workgroup per (key block, KV head), looping over the KV head's
//              G query heads with dK and dV in registers: the reduction over the heads
//              happens on chip (section 6.5), in a fixed order, so results are
//              deterministic and no partial sums go through memory.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 32 keys x 32 query rows per wave step):
//   dq kernel   S^T = K.Q^T and dP^T = V.dO^T (K, V rows from LDS; Q, dO fragments in
//               registers); a lane owns one query row, so LSE and D are per-lane scalars;
//               dQ^T += K^T.dS^T takes dS^T straight from the score registers (B operand)
//               and K^T through the LDS transpose read.
//   dkdv kernel S = Q.K^T and dP = dO.V^T (Q, dO rows from LDS; K and V rows from the
//               workgroup's K and V blocks in LDS); a lane owns one key;
//               dV^T += dO^T.P and dK^T += Q^T.dS take P and dS straight from the score
//               registers and dO^T, Q^T through the LDS transpose read.
// Tiles that are read both by rows and transposed store 16-byte chunk c of row r at chunk
// position c ^ (4 (r % 4) + (r / 4) % 4): sixteen consecutive rows then fall on sixteen
// distinct positions (row reads), and so do four consecutive rows of one 64-byte column
// group (transpose reads).
#include <type_traits>

#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int D = 128;
constexpr int kRowBytes = D * 2;               // one row of one head: 256 bytes
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStatRows = 64;                  // rows per statistics block
constexpr int kStatFloats = 2 * kStatRows;     // lse2 then D

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Buffer-resource word 3 of the gfx9 family (32-bit data format, no swizzle).
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// DMA of 32 consecutive rows (each 256 bytes, row_bytes apart, the first at gbase) into LDS
// at lds + dst in the swizzled layout.  Wave w copies rows 4w .. 4w+3: lane l lands at row
// 4w + l/16, chunk position l%16, and fetches the logical chunk stored there (voff is that
// chunk's byte offset from the group's first row).  Only the first `rows` rows are read;
// the others arrive as zeros and cost no memory traffic.
__device__ __forceinline__ void dma_rows32(uint8_t *lds, int dst, const uint16_t *gbase,
                                           uint32_t row_bytes, int rows, uint32_t voff, int w) {
    uint32_t bytes = rows <= 0 ? 0u : rows >= 32 ? 32u * row_bytes : (uint32_t)rows * row_bytes;
    bytes = __builtin_amdgcn_readfirstlane(bytes);
    const uint64_t base = (uint64_t)gbase;
    const u32x4 rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, kRsrcWord3};
    const uint32_t lds_dst = (uint32_t)(uintptr_t)(lds + dst + 4 * w * kRowBytes);
    // (assembly, so that the compiler adds no wait for the DMA before later LDS reads: the
    // loops' own waits and barriers order the buffers)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory");
}

// DMA of up to 1 KiB of contiguous bytes (the first `bytes` of them real, the rest zeros)
// into lds + dst: lane l's 16 bytes land at dst + 16 l.
__device__ __forceinline__ void dma_bytes1k(uint8_t *lds, int dst, const void *gbase,
                                            uint32_t bytes, uint32_t voff) {
    bytes = __builtin_amdgcn_readfirstlane(bytes);
    const uint64_t base = (uint64_t)gbase;
    const u32x4 rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, kRsrcWord3};
    const uint32_t lds_dst = (uint32_t)(uintptr_t)(lds + dst);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_dst))
                 : "memory");
}

// Per-lane LDS byte offsets, fixed for a kernel's life.
//   row[ks]: the 16 bytes of row lane%32 (relative to a 32-row group) that hold reduction
//            slots d = 16 ks + 8 (lane/32) .. +7 (an A or B operand read along d);
//   tr[dt][m&1]: the transpose-read start for column group dt (d = 32 dt ..) at row
//            offset 8m of a 32-row group; rows 16 kk further add 16 kk rows.
struct Addr {
    uint32_t row[8];
    uint32_t tr[4][2];
};

__device__ __forceinline__ Addr make_addr(int lane) {
    Addr a;
    const int r32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        a.row[ks] = (uint32_t)(r32 * kRowBytes + 16 * ((2 * ks + hf) ^ swz(r32)));
    // transpose read: lane j of each 16-lane group points at row 4hf + (j%16)/4, 8 bytes
    // at column 4 (j%4) of its 16-column half of the 64-byte group (see lds_read_tr16)
    const int vr = 4 * hf + ((lane & 15) >> 2);
    const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        a.tr[dt][0] = (uint32_t)(vr * kRowBytes + 16 * ((4 * dt + cc) ^ swz(vr)) + 8 * (lane & 1));
        // row vr + 8: swz(vr + 8) = swz(vr) ^ 2, i.e. the chunk index with bit 1 flipped
        a.tr[dt][1] = (uint32_t)((vr + 8) * kRowBytes +
                                 16 * ((4 * dt + cc) ^ swz(vr + 8)) + 8 * (lane & 1));
    }
    return a;
}

// The 8-slot operand of reduction rows 16 kk + {8 (j/4) + 4 hf + j%4} of column lane%32
// of column group dt, from a swizzled 32-row group at lds + base: two transpose reads
// (rows 4hf.. and 8 + 4hf..).  Rows 16 further have the same swizzle (swz(r + 16) = swz(r)).
__device__ __forceinline__ bf16x8 read_tr(const uint8_t *lds, uint32_t base, const Addr &a,
                                          int dt, int kk) {
    const uint8_t *p0 = lds + base + a.tr[dt][0] + kk * 16 * kRowBytes;
    const uint8_t *p1 = lds + base + a.tr[dt][1] + kk * 16 * kRowBytes;
    const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(p0));
    const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(p1));
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ bf16x8 read_row(const uint8_t *lds, uint32_t base, const Addr &a,
                                           int ks) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(lds + base + a.row[ks]));
}

// Elements 8 kk .. 8 kk + 7 of a lane's 16 scores as a bf16 B operand (reduction slot j <->
// element 8 kk + j, the order the transpose reads deliver the other operand in).
__device__ __forceinline__ bf16x8 pack8(const float (&x)[16], int kk) {
    const u32x4 w = {pack_bf16x2(x[8 * kk + 0], x[8 * kk + 1]), pack_bf16x2(x[8 * kk + 2], x[8 * kk + 3]),
                     pack_bf16x2(x[8 * kk + 4], x[8 * kk + 5]), pack_bf16x2(x[8 * kk + 6], x[8 * kk + 7])};
    return as_bf16x8(w);
}

// ---------------------------------------------------------------------------------------
// bwd_prep: one row (b, h, i) per 16 lanes, i over the padded length n_t * 64.

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a, int n_t) {
    const int sub = threadIdx.x & 15;
    const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const long n_pad = (long)n_t * kStatRows;
    const long total = (long)a.B * a.H_q * n_pad;
    if (row >= total) return;   // (whole 16-lane groups leave together)
    const int i = (int)(row % n_pad);
    const long bh = row / n_pad;
    const int h = (int)(bh % a.H_q), b = (int)(bh / a.H_q);
    float dot = 0.f;
    if (i < a.S) {
        const size_t off = (((size_t)b * a.S + i) * a.H_q + h) * D + sub * 8;
        const bf16x8 o = as_bf16x8(load16(a.o + off));
        const bf16x8 g = as_bf16x8(load16(a.dout + off));
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf((float)o[e], (float)g[e], dot);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 16);
    if (sub == 0) {
        float *blk = a.stats + (bh * n_t + i / kStatRows) * kStatFloats;
        // rows past the end: lse2 = +inf makes every P of the row 0, D = 0
        blk[i % kStatRows] =
            i < a.S ? a.lse[bh * a.S + i] * kLog2e : __builtin_inff();
        blk[kStatRows + i % kStatRows] = i < a.S ? dot : 0.f;
    }
}

// ---------------------------------------------------------------------------------------
// bwd_dq: workgroup = 256 query rows of one query head (8 waves x 32 rows), key tiles of 64
// through a ring of two LDS slots (K 16 KiB, V 16 KiB each); the tile loop is unrolled by two
// so that each slot's fragment offsets are compile-time immediates.

constexpr int kQBr = 256;
constexpr int kKT = 64;
constexpr int kTile = kKT * kRowBytes;               // 16 KiB
constexpr int kDqSlot = 2 * kTile;                   // K then V
constexpr int kDqLds = 2 * kDqSlot;                  // 64 KiB

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a, int n_qb, int n_t) {
    __shared__ __attribute__((aligned(256))) uint8_t smem[kDqLds];
    const int G = a.H_q / a.H_kv;
    int u = blockIdx.x;
    const int h = u % a.H_q;
    u /= a.H_q;
    const int b = u % a.B;
    const int qb = n_qb - 1 - u / a.B;     // long-prefix blocks first
    const int g = h / G;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, hf = lane >> 5;
    const int i0 = qb * kQBr;
    const int r0 = i0 + 32 * w;            // the wave's first row
    const int row = r0 + r32;              // the lane's row
    const int last_row = min(i0 + kQBr, a.S) - 1;
    const int n_kt = last_row / kKT + 1;   // key tiles of the workgroup
    // 32-key steps of the wave (up to its last real row's diagonal); the step holding row
    // r0's diagonal and the ones after it are masked
    const int n_sub = r0 < a.S ? min(r0 + 31, a.S - 1) / 32 + 1 : 0;
    const int mask_from = r0 / 32;
    const Addr ad = make_addr(lane);

    const uint32_t kv_row_bytes = (uint32_t)a.H_kv * kRowBytes;
    const uint16_t *kbase = a.k + ((size_t)b * a.S * a.H_kv + g) * D;
    const uint16_t *vbase = a.v + ((size_t)b * a.S * a.H_kv + g) * D;
    const int lr = 4 * w + lane / 16;
    const uint32_t voff = (uint32_t)lr * kv_row_bytes + 16u * (uint32_t)((lane & 15) ^ swz(lr));

    // Q and dO fragments (B operands): column = the lane's row, slots d = 16 ks + 8 hf ..
    bf16x8 qf[8], gf[8];
    {
        const int rr = min(row, a.S - 1);
        const size_t off = (((size_t)b * a.S + rr) * a.H_q + h) * D + hf * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks] = as_bf16x8(load16(a.q + off + 16 * ks));
            gf[ks] = as_bf16x8(load16(a.dout + off + 16 * ks));
        }
    }
    const float *st = a.stats + (((size_t)b * a.H_q + h) * n_t + min(row, a.S - 1) / kStatRows) *
                                    kStatFloats;
    const float lse2 = st[min(row, a.S - 1) % kStatRows];
    const float Drow = st[kStatRows + min(row, a.S - 1) % kStatRows];
    const float c = a.scale_log2;

    f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

    auto issue = [&](int t, int slot) {
        const int k0 = t * kKT;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = k0 + 32 * i;
            dma_rows32(smem, slot * kDqSlot + 32 * i * kRowBytes, kbase + (size_t)r * a.H_kv * D,
                       kv_row_bytes, a.S - r, voff, w);
            dma_rows32(smem, slot * kDqSlot + kTile + 32 * i * kRowBytes,
                       vbase + (size_t)r * a.H_kv * D, kv_row_bytes, a.S - r, voff, w);
        }
    };

    // one key tile t in ring slot SLOT = t % 2, a compile-time constant so that every LDS
    // fragment address is a fixed per-lane register plus an immediate offset
    auto tile = [&](int t, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        issue(t + 1, slot ^ 1);   // (past the last tile it only zero-fills the free slot)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int us = 2 * t + hh;
            if (us >= n_sub) continue;
            const uint32_t kh = slot * kDqSlot + hh * 32 * kRowBytes;
            const uint32_t vh = kh + kTile;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                s = mfma32(read_row(smem, kh, ad, ks), qf[ks], s);
                dp = mfma32(read_row(smem, vh, ad, ks), gf[ks], dp);
            }
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = exp2_fast(fmaf(s[r], c, -lse2));
            if (us >= mask_from) {
                // a step holding the wave's diagonal: keys past the lane's row get no weight
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * us + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > row) p[r] = 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[r] - Drow);
            const bf16x8 d0 = pack8(ds, 0), d1 = pack8(ds, 1);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                acc[dt] = mfma32(read_tr(smem, kh, ad, dt, 0), d0, acc[dt]);
                acc[dt] = mfma32(read_tr(smem, kh, ad, dt, 1), d1, acc[dt]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // the next tile's DMA
        __syncthreads();
    };

    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int t = 0;
    for (; t + 1 < n_kt; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        tile(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < n_kt) tile(t, std::integral_constant<int, 0>{});

    // dQ times tau; every tile ended with a barrier after its DMA landed, so the rings are
    // free for the staging
    static_assert(kWaves * 32 * kRowBytes <= kDqLds, "each wave stages its 32 rows");
    store_rows128(acc, a.scale, smem + w * (32 * kRowBytes), a.dq + ((size_t)b * a.S * a.H_q + h) * D,
               (size_t)a.H_q * D, r0, a.S, lane);
}

// ---------------------------------------------------------------------------------------
// bwd_dkdv: workgroup = one block of 128 keys of one KV head against the rows of all G query
// heads of that KV head, with dK and dV accumulated in registers over the heads: the
// reduction over a KV head's query heads happens on chip (V07 section 6.5), nothing but the
// row statistics goes through memory, and the order of the additions is fixed.  Wave w takes
// the 32 keys of key group w % 4 and, of each 64-row query tile, the 32 rows of row half
// w / 4; the two waves of a SIMD (waves are dealt to SIMDs round-robin) thus share their keys
// and split the rows of every tile, and at the end the second half's dK and dV are added to
// the first's through LDS.  Blocks with the longest prefix of rows run first.  A work item is
// a (query tile, head) pair, heads inner.
// The two halves run an item out of phase: row half 1 forms the dV / dK products of an item
// one item late, at the start of the next, so that while row half 0 runs an item's softmax
// arithmetic the other wave of its SIMD keeps the matrix core busy (with the items in step,
// both waves of a SIMD would reach their softmax together, and the matrix core would idle).
// Each half therefore DMAs only its own 32 rows of a tile, into a ring of its own: two slots
// for half 0, three for half 1, whose late products still read an item's slot while the next
// item's DMA goes out.  LDS: the block's V rows (32 KiB) and K rows (32 KiB), then the two
// rings of slots of a half tile of one head (Q 8 KiB, dO 8 KiB, the tile's statistics block
// 1 KiB), then 1 KiB that the other waves' statistics DMA fills with zeros.

constexpr int kKBlk = 128;                           // keys per workgroup
constexpr int kVBlock = kKBlk * kRowBytes;           // 32 KiB
constexpr int kKBlock = kVBlock;                     // the block's K rows after its V rows
constexpr int kHalfTile = 32 * kRowBytes;           // 8 KiB: one row half of a query tile
constexpr int kSlot = 2 * kHalfTile + 1024;          // Q, dO half tiles, statistics block
constexpr int kRing = kVBlock + kKBlock;             // row half 0: slots 0, 1
constexpr int kRing1 = kRing + 2 * kSlot;            // row half 1: slots 0, 1, 2
constexpr int kSink = kRing1 + 3 * kSlot;
constexpr int kKvLds = kSink + 1024;                 // 150 KiB: one workgroup per CU

// Row half 1 stores its accumulators x at xch (element 4 j .. 4 j + 3 at xch[64 j]); row
// half 0 adds them to its own (half 0 + half 1, a fixed order).  Both halves call it.
__device__ __forceinline__ void hand_over(f32x16 (&x)[4], f32x4 *xch, int rh) {
    if (rh == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xch[(dt * 4 + q) * 64] =
                    f32x4{x[dt][4 * q], x[dt][4 * q + 1], x[dt][4 * q + 2], x[dt][4 * q + 3]};
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 y = xch[(dt * 4 + q) * 64];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[dt][4 * q + e] += y[e];
            }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a, int n_t) {
    __shared__ __attribute__((aligned(256))) uint8_t smem[kKvLds];
    const int G = a.H_q / a.H_kv;
    int u = blockIdx.x;
    const int g = u % a.H_kv;
    u /= a.H_kv;
    const int b = u % a.B;
    const int kb = u / a.B;                          // block 0 (every row sees it) first

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, hf = lane >> 5;
    const int rh = w / 4, kg = w % 4;                // row half, key group
    const int k0 = kb * kKBlk;
    const int kw0 = k0 + 32 * kg;                    // the wave's first key (lane: kw0 + r32)
    const int t0 = k0 / kStatRows;                   // first query tile: rows k0 ..
    const Addr ad = make_addr(lane);
    const int lr = 4 * w + lane / 16;

    const uint32_t q_row_bytes = (uint32_t)a.H_q * kRowBytes;
    const uint32_t kv_row_bytes = (uint32_t)a.H_kv * kRowBytes;
    const uint32_t kvvoff = (uint32_t)lr * kv_row_bytes + 16u * (uint32_t)((lane & 15) ^ swz(lr));
    // a row half's own rows: wave kg copies row quads kg and kg + 4 of its 32-row half (the
    // swizzle of a row depends on its row % 16 only, so both quads share the lane's chunk)
    const int lq = 4 * kg + lane / 16;
    const uint32_t qvoff = (uint32_t)lq * q_row_bytes + 16u * (uint32_t)((lane & 15) ^ swz(lq));

    // the block's V and K rows: each wave copies 4 rows of every 32-row group
    {
        const size_t off = (((size_t)b * a.S + k0) * a.H_kv + g) * D;
#pragma unroll
        for (int i = 0; i < kKBlk / 32; ++i) {
            dma_rows32(smem, 32 * i * kRowBytes, a.v + off + (size_t)32 * i * a.H_kv * D,
                       kv_row_bytes, a.S - k0 - 32 * i, kvvoff, w);
            dma_rows32(smem, kVBlock + 32 * i * kRowBytes, a.k + off + (size_t)32 * i * a.H_kv * D,
                       kv_row_bytes, a.S - k0 - 32 * i, kvvoff, w);
        }
    }
    const uint32_t vrow = 32u * kg * kRowBytes;              // the wave's V rows in the block
    const uint32_t krow = kVBlock + vrow;                    // and its K rows

    const int n_items = (n_t - t0) * G;
    // items are (query tile, head) pairs, heads inner; the DMA side runs one item ahead of the
    // compute side, and both step through the items by increments (no division per item)
    auto slot_base = [&](int par, int m3) {
        return rh == 0 ? kRing + par * kSlot : kRing1 + m3 * kSlot;
    };
    // the next item to issue: its tile, head index, position mod 3, and the element offsets
    // of its rows in Q / dO and of its statistics block
    int is_t = t0, is_j = 0, is_m3 = 0;
    const size_t q_tile_step = (size_t)kStatRows * a.H_q * D;
    const size_t st_head_step = (size_t)n_t * kStatFloats;
    size_t is_q = (((size_t)b * a.S + (size_t)t0 * kStatRows + 32 * rh) * a.H_q + (size_t)g * G) * D;
    size_t is_st = (((size_t)b * a.H_q + (size_t)g * G) * n_t + t0) * kStatFloats;
    // this wave's share of an item's DMA into its half's slot for the item: two row quads of
    // its half of the Q and dO tiles; the first wave of each half also the statistics
    // block, the other waves zero-fill the sink
    auto issue = [&](int it) {
        const bool real = it < n_items;
        const int base = slot_base(it & 1, is_m3);
        const int r = is_t * kStatRows + 32 * rh;
        const int rows = real ? a.S - r : 0;          // past the last item: zero-fill only
        const uint16_t *qbase = a.q + is_q;
        const uint16_t *gbase = a.dout + is_q;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            dma_rows32(smem, base, qbase, q_row_bytes, rows, qvoff + 16u * i * q_row_bytes,
                       kg + 4 * i);
            dma_rows32(smem, base + kHalfTile, gbase, q_row_bytes, rows,
                       qvoff + 16u * i * q_row_bytes, kg + 4 * i);
        }
        // the statistics block (both halves' rows) by the first wave of each half
        const bool mine = kg == 0 && real;
        dma_bytes1k(smem, mine ? base + 2 * kHalfTile : kSink, a.stats + is_st,
                    mine ? (uint32_t)(kStatFloats * sizeof(float)) : 0u, 16u * (uint32_t)lane);
        if (++is_j == G) {
            is_j = 0;
            ++is_t;
            is_q += q_tile_step - (size_t)(G - 1) * D;
            is_st += kStatFloats - (size_t)(G - 1) * st_head_step;
        } else {
            is_q += D;
            is_st += st_head_step;
        }
        if (++is_m3 == 3) is_m3 = 0;
    };

    f32x16 dv[4], dk[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[dt][r] = dk[dt][r] = 0.f;
    const float c = a.scale_log2;

    bf16x8 p0 = {}, p1 = {}, d0 = {}, d1 = {};
    bool pend = false;                  // row half 1: an item's dV / dK products are owed
    uint32_t pqh = 0;
    auto dvdk = [&](uint32_t qh) {
        const uint32_t gh = qh + kHalfTile;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            dv[dt] = mfma32(read_tr(smem, gh, ad, dt, 0), p0, dv[dt]);
            dv[dt] = mfma32(read_tr(smem, gh, ad, dt, 1), p1, dv[dt]);
            dk[dt] = mfma32(read_tr(smem, qh, ad, dt, 0), d0, dk[dt]);
            dk[dt] = mfma32(read_tr(smem, qh, ad, dt, 1), d1, dk[dt]);
        }
    };

    issue(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int cu_t = t0, cu_j = 0, cu_m3 = 0;   // the compute side's item: tile, head index, it % 3
    for (int it = 0; it < n_items; ++it) {
        // row half 1: item it - 1's products first (its slot is not refilled until item
        // it + 2's DMA, after the barrier that ends item it)
        if (rh == 1 && pend) dvdk(pqh);
        issue(it + 1);
        const int r0 = cu_t * kStatRows + 32 * rh;            // the wave's first row
        pend = r0 >= kw0;                                     // (rows all before the keys: skip)
        if (pend) {
            const uint32_t qh = slot_base(it & 1, cu_m3);
            const uint32_t gh = qh + kHalfTile;
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                s = mfma32(read_row(smem, qh, ad, ks), read_row(smem, krow, ad, ks), s);
                dp = mfma32(read_row(smem, gh, ad, ks), read_row(smem, vrow, ad, ks), dp);
            }
            // lse2 and D of the lane's 16 rows 32 rh + 8 q + 4 hf + (0..3)
            const uint8_t *stp = smem + qh + 2 * kHalfTile;
            float p[16], ds[16];
            f32x4 d4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int rr = 32 * rh + 8 * q4 + 4 * hf;
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(stp + 4 * rr);
                d4[q4] = *reinterpret_cast<const f32x4 *>(stp + 4 * (kStatRows + rr));
#pragma unroll
                for (int j = 0; j < 4; ++j) p[4 * q4 + j] = exp2_fast(fmaf(s[4 * q4 + j], c, -l4[j]));
            }
            if (r0 == kw0) {
                // the diagonal step: rows r0 + (8 q4 + 4 hf + j), keys r0 + r32
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (r32 > 8 * q4 + 4 * hf + j) p[4 * q4 + j] = 0.f;
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int j = 0; j < 4; ++j) ds[4 * q4 + j] = p[4 * q4 + j] * (dp[4 * q4 + j] - d4[q4][j]);
            p0 = pack8(p, 0);
            p1 = pack8(p, 1);
            d0 = pack8(ds, 0);
            d1 = pack8(ds, 1);
            pqh = qh;
            if (rh == 0) dvdk(qh);
        }
        if (++cu_j == G) {
            cu_j = 0;
            ++cu_t;
        }
        if (++cu_m3 == 3) cu_m3 = 0;
        __builtin_amdgcn_s_waitcnt(0);   // the next item's DMA
        __syncthreads();
    }
    if (rh == 1 && pend) dvdk(pqh);      // the last item's
    __syncthreads();

    // row half 1 hands its sums to row half 0 through LDS (the query-tile rings, free now),
    // dK then dV: element 4 j .. 4 j + 3 of lane l of key group k at ((k * 16 + j) * 64 + l)
    // * 16 bytes, so each store and load of a wave is 1 KiB contiguous
    f32x4 *xch = reinterpret_cast<f32x4 *>(smem + kRing) + kg * 16 * 64 + lane;
    hand_over(dk, xch, rh);
    hand_over(dv, xch, rh);
    if (rh == 1) return;

    // dK (times tau) and dV of the wave's keys, summed over the G heads, rounded to bf16, staged
    // in the block's K/V buffers (free since the hand-over's barriers), 16 KiB per key group
    const size_t kvo = ((size_t)b * a.S * a.H_kv + g) * D;
    static_assert(4 * 64 * kRowBytes <= kRing, "the four key groups stage in the K/V block");
    uint8_t *stage = smem + kg * (64 * kRowBytes);
    store_rows128(dk, a.scale, stage, a.dk + kvo, (size_t)a.H_kv * D, kw0, a.S, lane);
    store_rows128(dv, 1.f, stage + 32 * kRowBytes, a.dv + kvo, (size_t)a.H_kv * D, kw0, a.S, lane);
}

}  // namespace

size_t prefill_bwd_workspace_bytes(int B, int S, int H_q) {
    const size_t n_t = (size_t)(S + kStatRows - 1) / kStatRows;
    return (size_t)B * H_q * n_t * kStatFloats * sizeof(float);
}

hipError_t launch_prefill_bwd(BwdArgs a, void *ws, hipStream_t stream) {
    if (a.d != D) return hipErrorInvalidValue;
    const int n_t = (a.S + kStatRows - 1) / kStatRows;
    const int n_qb = (a.S + kQBr - 1) / kQBr;
    a.stats = static_cast<float *>(ws);

    const long prep_rows = (long)a.B * a.H_q * n_t * kStatRows;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((prep_rows + 15) / 16)), dim3(256), 0,
                       stream, a, n_t);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((long)n_qb * a.B * a.H_q)), dim3(kThreads),
                       0, stream, a, n_qb, n_t);
    const int n_kb = (a.S + kKBlk - 1) / kKBlk;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)((long)n_kb * a.B * a.H_kv)),
                       dim3(kThreads), 0, stream, a, n_t);
    return hipGetLastError();
}

}  // namespace gqa
