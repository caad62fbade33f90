// prefill_causal.hip -- causal GQA prefill on gfx950: a whole prompt (T_q = S_kv), or a
// chunk of T_q query rows that are the tokens q_start .. q_start + T_q - 1 of a sequence
// whose keys are cached (ADR-0060 "AHBM GQA Fused Attention", section 0.5.2: the launch
// carries the query block's q_start and T_q; section 5.4: the query block against the
// KV tiles, past / future / partial).  Query row i sees keys j <= q_start + i.
//
// FlashAttention-2 forward ("Attention Kernel lineage" (V07), sections 7-8):
// each workgroup owns one block of 256 query rows of one query head for its
// whole life (8 waves of 32 rows, one workgroup per CU), keeps the rows'
// (m, l, O) state in registers, and streams 64-key K/V tiles through LDS; the
// division by l is deferred to the end, and the score matrix is never written
// (section 4).  Causal block classification (section 12): a tile wholly above
// the diagonal is never loaded, and only keys crossing the diagonal are masked.
// The classification is applied per wave in 32-key steps: a wave stops after the
// step holding its own diagonal, and only that step's scores are masked (to -inf,
// when they are formed one step earlier), so every step runs the same code.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16): scores are formed
// transposed, S^T = K . Q^T, so each lane owns one query row (lane % 32) and
// holds 16 of that row's 32 scores of a step; the row max and sum need one
// cross-lane step.  P.V is formed as O^T = V^T . P^T, whose B operand is exactly
// the softmax output registers, and whose accumulator keeps one query row per
// lane, so the rescale by alpha is a per-lane scalar.  Q (B operand) stays in
// registers; the K fragments are 16-byte LDS reads; V^T fragments (8 keys of one
// d column) come from the row-major V tile through the LDS transpose read.
//
// Software pipeline inside each wave (32-key steps): the matrix cores form the
// scores of step u+1 while the vector units run the softmax of step u (V07 section
// 10 overlaps the same two phases across warpgroups).  A step first issues all of its
// LDS fragment reads -- the K rows of step u+1 and the V^T fragments of step u -- so
// that no product waits for LDS in the middle of the step.  The softmax runs against
// the running max as it stands; only when a step's P passes a bound (a score above the
// running max by about 8 in log2 units, and always on the first step) is the max
// raised to the row's maximum and the step formed again, so the common step takes no
// row maximum at all (V07 section 3: any common shift cancels in O / l).  K/V tiles travel from HBM
// straight into LDS (buffer loads with an LDS destination: no staging
// registers; rows past the sequence end read as zeros) through rings of four K
// and four V tile buffers, each tile issued three tiles ahead of its use.
// Rows are stored with their 16-byte chunks XOR-permuted so that the fragment
// reads of both products are bank-conflict free without padding.
//
// Scores are kept in log2 units (s2 = acc * tau * log2(e), one fp32 multiply
// folded into the exponent's FMA; V07 section 2, exp2 trick).
//
// Paged cache (the Paged instantiation; V07 sections 16-17, block table and pool): the
// sequence's block-table row is staged in LDS when the workgroup starts; each DMA instruction
// of a tile covers four consecutive rows of one page, whose pool row a wave looks up once per
// tile and uses for both the K and the V DMA of that tile (K and V pools share the table);
// the tiles land in LDS exactly as from a contiguous cache, so the arithmetic is the same.
//
// Grid: one workgroup per (q-block, sequence, query head), heaviest q-blocks
// first (V07 section 12, causal-aware scheduling).  Consecutive workgroups are
// dispatched round-robin over the 8 XCDs; the index is remapped so that the G
// query heads sharing one KV head and q-block run back to back on one XCD and
// hit its L2 for the shared K/V tiles (V07 section 14: K/V loaded once, reused
// by the group).
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {
namespace {

constexpr int D = 128;
constexpr int kBr = 256;          // query rows per workgroup
constexpr int kBc = 64;           // keys per LDS tile
constexpr int kHalf = 32;         // keys per pipeline step (half a tile)
constexpr int kWaves = 8;         // 32 query rows per wave, two waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = D * 2;                  // one key row of one head: 256 B
constexpr int kTileBytes = kBc * kRowBytes;       // 16 KiB
constexpr int kNK = 4;                            // LDS: a ring of four K tile buffers
constexpr int kNV = 4;                            // and a ring of four V tile buffers
constexpr int kKBuf = 0;
constexpr int kVBuf = kNK * kTileBytes;
constexpr int kLdsBytes = (kNK + kNV) * kTileBytes;   // 128 KiB: one workgroup per CU
constexpr int kDmaPerTile = 2;                    // DMA instructions per wave, tile and tensor
constexpr int kXcds = 8;
constexpr float kPBound = 256.f;   // a lane's step sum of P above this moves the running max

typedef __attribute__((address_space(3))) void lds_void;

// LDS row layouts (16-byte chunk c of row r lives at chunk position c ^ f(r)):
//   K: f(r) = r % 16   -- the QK fragment read has 16 consecutive rows read the same
//                         chunk in one pass, which then fall on 16 distinct positions;
//   V: f(r) = 4 (r % 4) -- a transpose read covers 4 consecutive rows x 4 chunks of one
//                         64-byte column group, which then fill all 16 positions.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

// Issue the DMA of one 64-row K or V tile (keys k0..k0+63) into the LDS buffer at byte
// offset dst.  Wave w writes rows 32i + 4w .. +3 (i = 0, 1); its lane l lands at row
// 32i + 4w + l/16, chunk position l%16, and fetches the chunk the layout puts there
// (voff: that chunk's byte offset from key row 32i).  Each 32-row group gets its own
// buffer range, ending at the sequence end, so rows past it arrive as zeros (a tile
// wholly past the end costs no memory traffic and just zero-fills its buffer).
__device__ __forceinline__ void dma_tile(uint8_t *lds, int dst, const uint16_t *gbase,
                                         size_t kv_row, int k0, int S, uint32_t voff, int w) {
    const uint32_t row_bytes = (uint32_t)kv_row * 2u;
    const bool full = k0 + kBc <= S;   // every tile but the last ones
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        const int r0 = k0 + 32 * i;
        uint32_t bytes = 32u * row_bytes;
        if (!full) {
            const int rows = S - r0;
            bytes = rows <= 0 ? 0u : rows >= 32 ? bytes : (uint32_t)rows * row_bytes;
        }
        // (uniform; readfirstlane keeps the resource in scalar registers)
        bytes = __builtin_amdgcn_readfirstlane(bytes);
        const uint64_t base = (uint64_t)(gbase + (size_t)r0 * kv_row);
        // buffer resource: base, stride 0, range `bytes`, gfx9 data format word
        const u32x4 rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, 0x00020000u};
        const uint32_t lds_dst = (uint32_t)(uintptr_t)(lds + dst + (32 * i + 4 * w) * kRowBytes);
        // Issued as assembly so that the compiler does not add a wait for this DMA before
        // every later LDS read: the tile loop's own waits and barriers order the buffers.
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_dst))
                     : "memory");
    }
}

// The same DMA from a paged cache: wave w's four rows r .. r + 3 (r = k0 + 32 i + 4 w, a
// multiple of 4) lie in one page, since pages hold a multiple of 16 rows, so each DMA
// instruction reads from one page: row r % page of page tbl[r / page] (the sequence's table
// row, staged in LDS), its lane l fetching row l / 16 of the four and the chunk the layout
// puts at position l % 16 (voff).  Rows at or past S, and pages outside the pool, arrive as
// zeros and are not read.
__device__ __forceinline__ void dma_tile_paged(uint8_t *lds, int dst, const uint16_t *pool,
                                               size_t kv_row, int k0, int S, uint32_t voff, int w,
                                               const int *tbl, int page, int num_pages) {
    const uint32_t row_bytes = (uint32_t)kv_row * 2u;
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        const int r = k0 + 32 * i + 4 * w;
        uint32_t bytes = 0;
        uint64_t base = (uint64_t)pool;
        if (r < S) {
            const int pg = __builtin_amdgcn_readfirstlane(tbl[r / page]);
            if ((unsigned)pg < (unsigned)num_pages) {
                bytes = (uint32_t)min(4, S - r) * row_bytes;
                base = (uint64_t)(pool + ((size_t)pg * page + r % page) * kv_row);
            }
        }
        bytes = __builtin_amdgcn_readfirstlane(bytes);
        const u32x4 rsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) & 0xFFFFu,
                            bytes, 0x00020000u};
        const uint32_t lds_dst = (uint32_t)(uintptr_t)(lds + dst + (32 * i + 4 * w) * kRowBytes);
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_dst))
                     : "memory");
    }
}

// Per-lane LDS byte offsets of the fragment reads, fixed for the kernel's life.
struct FragAddr {
    uint32_t k[8];   // K: row r32, chunk hf*8 + k8, from a half tile's first row
    uint32_t v[4];   // V: transpose-read start for d tile dt (add 16 rows per k-step)
};

// K fragments of 32 keys whose K rows start at LDS byte offset kh.
__device__ __forceinline__ void load_k(bf16x8 (&kf)[8], const uint8_t *kh, const FragAddr &fa) {
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8)
        kf[k8] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kh + fa.k[k8]));
}

// S^T = K . Q^T for 32 keys.
__device__ __forceinline__ void qk_half(f32x16 &s, const bf16x8 (&kf)[8], const bf16x8 (&qf)[8]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) s = mfma32(kf[k8], qf[k8], s);
}

// S^T = K . Q^T for 32 keys whose K rows start at LDS byte offset kh.
__device__ __forceinline__ void qk_half(f32x16 &s, const uint8_t *kh, const FragAddr &fa,
                                        const bf16x8 (&qf)[8]) {
    bf16x8 kf[8];
    load_k(kf, kh, fa);
    qk_half(s, kf, qf);
}

// Element r of a lane's 16 scores of a half is key k0 + 8*(r/4) + 4*hf + r%4.
__device__ __forceinline__ int score_key(int k0, int r, int hf) {
    return k0 + (r >> 2) * 8 + hf * 4 + (r & 3);
}

// P = 2^(s * c - m) as the B operand of P.V (a masked score, -inf, gives 0), with the
// step's two row sums of this lane's half: rs of the fp32 P, rw of the bf16-rounded P.
__device__ __forceinline__ void softmax_half(const f32x16 &s, float m, float c,
                                             bf16x8 (&pf)[2], float &rs_out, float &rw_out) {
    const float neg_m = -m;
    float rs = 0.f, rw = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = exp2_fast(fmaf(s[kk * 8 + j], c, neg_m));
            rs += p[j];
        }
        const u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                         pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
        for (int i = 0; i < 4; ++i) rw = add_bf16_pair(w[i], rw);
        pf[kk] = as_bf16x8(w);
    }
    rs_out = rs;
    rw_out = rw;
}

// New running max after a step whose P overflowed the bound (or the first step, m = -inf):
// m = the row's max of m and its scores (both lanes of the row agree), and O, l rescaled.
__device__ __forceinline__ void raise_max(const f32x16 &s, float c, float &m, float &l, float &lw,
                                          f32x16 (&o)[4]) {
    float mx = neg_inf();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx * c);
    const float alpha = exp2_fast(m - m_new);     // 0 on the first step
    l *= alpha;
    lw *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m = m_new;
}

// V^T fragments of 32 keys whose V rows start at LDS byte offset vh: for d tile dt and
// k-step kk, the two transpose reads that make one 8-key operand.  Read all at once, ahead
// of the softmax, so that the P.V products never wait for LDS.
struct VtFrags {
    u32x4 f[4][2];
};

__device__ __forceinline__ void load_vt(VtFrags &vt, const uint8_t *vh, const uint32_t (&va)[4]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const uint8_t *vp = vh + va[dt] + kk * 16 * kRowBytes;
            const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(vp));
            const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(vp + 8 * kRowBytes));
            vt.f[dt][kk] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }
}

// O^T += V^T . P^T over 32 keys.
__device__ __forceinline__ void pv_half(f32x16 (&o)[4], const VtFrags &vt, const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) o[dt] = mfma32(as_bf16x8(vt.f[dt][kk]), pf[kk], o[dt]);
}

struct WaveCtx {
    uint8_t *lds;
    const uint16_t *kbase, *vbase;
    size_t kv_row;
    int S;                    // keys that may be read: q_start + T (the rest read as zeros)
    int n_kb, n_sub;          // LDS tiles of the workgroup, 32-key steps of this wave
    int mask_from;            // first step holding a key past some row's diagonal
    int w, row, hf;           // row: this lane's query position q_start + i
    float c;
    uint32_t koff, voff;   // DMA: this lane's byte offset within its 32-row group (paged:
                           // within its wave's four rows)
    FragAddr fa;
    const int *tbl;        // paged: the sequence's block-table row, in LDS
    int page, num_pages;
};

// One K or V tile DMA, from the contiguous cache or through the block table.
template <bool Paged>
__device__ __forceinline__ void dma(const WaveCtx &x, int dst, const uint16_t *base, int k0,
                                    uint32_t off) {
    if constexpr (Paged)
        dma_tile_paged(x.lds, dst, base, x.kv_row, k0, x.S, off, x.w, x.tbl, x.page, x.num_pages);
    else
        dma_tile(x.lds, dst, base, x.kv_row, k0, x.S, off, x.w);
}

// Paged: the pool rows of one tile's DMA for this wave (its rows 32 i + 4 w .. + 3 of the
// tile lie in one page), looked up once and used for both the K and the V DMA of the tile.
struct PageRows {
    size_t row[kDmaPerTile];       // first pool row, in elements (0 when nothing is read)
    uint32_t bytes[kDmaPerTile];   // bytes to read (0: zeros)
};

__device__ __forceinline__ PageRows page_rows(const WaveCtx &x, int k0) {
    PageRows p;
    const uint32_t row_bytes = (uint32_t)x.kv_row * 2u;
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        const int r = k0 + 32 * i + 4 * x.w;
        uint32_t bytes = 0;
        size_t row = 0;
        if (r < x.S) {
            const int pg = __builtin_amdgcn_readfirstlane(x.tbl[r / x.page]);
            if ((unsigned)pg < (unsigned)x.num_pages) {
                bytes = (uint32_t)min(4, x.S - r) * row_bytes;
                row = ((size_t)pg * x.page + r % x.page) * x.kv_row;
            }
        }
        p.row[i] = row;
        p.bytes[i] = __builtin_amdgcn_readfirstlane(bytes);
    }
    return p;
}

// The paged DMA of one tile from precomputed pool rows (the same loads as dma_tile_paged).
__device__ __forceinline__ void dma_rows_paged(const WaveCtx &x, int dst, const uint16_t *pool,
                                               const PageRows &p, uint32_t voff) {
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        const uint64_t base = (uint64_t)(pool + p.row[i]);
        const u32x4 rsrc = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) & 0xFFFFu,
                            p.bytes[i], 0x00020000u};
        const uint32_t lds_dst = (uint32_t)(uintptr_t)(x.lds + dst + (32 * i + 4 * x.w) * kRowBytes);
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_dst))
                     : "memory");
    }
}

struct RowState {
    f32x16 o[4];
    float m, l, lw;
};

// Scores of keys past the lane's query position become -inf (their P is then exactly 0).
__device__ __forceinline__ void mask_half(f32x16 &s, int k0, int row, int hf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = score_key(k0, r, hf) <= row ? s[r] : neg_inf();
}

// Pipeline step u (keys 32u .. 32u+31) of one wave, whose steps run 0 .. n_sub-1; steps
// from mask_from on hold the wave's diagonal (the last one, or the last two when the
// chunk start is not a multiple of 32), and their scores were masked when formed.
// The step runs its softmax while the matrix cores form the scores of step u+1 (K rows
// at kn), then its P.V (V rows at vh) while the row max of step u+1 is taken.  Every step
// runs the same code, the last one included (its scores for a step u+1 are not used).
__device__ __forceinline__ void half_step(const WaveCtx &x, int u, const f32x16 &s, f32x16 &sn,
                                          const uint8_t *kn, const uint8_t *vh,
                                          const uint32_t (&va)[4], const bf16x8 (&qf)[8],
                                          RowState &st) {
    if (u >= x.n_sub) return;
    bf16x8 kf[8];
    load_k(kf, kn, x.fa);
    VtFrags vt;
    load_vt(vt, vh, va);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pf[2];
    float rs, rw;
    softmax_half(s, st.m, x.c, pf, rs, rw);
    qk_half(sn, kf, qf);
    // the running max is moved only when a P of this step passes the bound (or is NaN, as on
    // the first step, where m = -inf): then the step is formed again against the new max
    if (__any(!(rs <= kPBound))) {
        raise_max(s, x.c, st.m, st.l, st.lw, st.o);
        softmax_half(s, st.m, x.c, pf, rs, rw);
    }
    st.l += rs;
    st.lw += rw;
    pv_half(st.o, vt, pf);
    // (masking the scores of step n_sub, which no step uses, is harmless)
    if (u + 1 >= x.mask_from) mask_half(sn, (u + 1) * kHalf, x.row, x.hf);
}

// One LDS tile kb (KI = kb % 4 names its K and V buffers).  Start the DMA of K(kb+3) into
// the K buffer that K(kb-1) has left, run the first pipeline step of tile kb, start the DMA
// of V(kb+3) into the V buffer V(kb-1) has left (issuing the two apart measured slightly
// faster than back to back), run the second step (which forms the scores of tile kb+1's
// first half); then wait for the DMA issued one tile earlier (K(kb+2) and V(kb+2)) and meet
// the other waves.  Every buffer written here is read at least two barriers later, and
// every buffer read here is refilled only after the next barrier.  The DMA is issued on
// every tile (past the end it only zero-fills a free buffer), so each wave has exactly
// 2 * kDmaPerTile of them per tile.
template <int KI, bool Paged>
__device__ __forceinline__ void tile_step(const WaveCtx &x, int kb, f32x16 &sa, f32x16 &sb,
                                          const bf16x8 (&qf)[8], RowState &st) {
    constexpr int kCur = kKBuf + KI * kTileBytes;
    constexpr int kNext = kKBuf + ((KI + 1) % kNK) * kTileBytes;
    constexpr int kFree = kKBuf + ((KI + 3) % kNK) * kTileBytes;
    constexpr int vcur = kVBuf + KI * kTileBytes;
    constexpr int vfree = kVBuf + ((KI + 3) % kNV) * kTileBytes;
    PageRows pr;
    if constexpr (Paged) {
        pr = page_rows(x, (kb + 3) * kBc);
        dma_rows_paged(x, kFree, x.kbase, pr, x.koff);
    } else {
        dma<Paged>(x, kFree, x.kbase, (kb + 3) * kBc, x.koff);
    }
    uint32_t va[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) va[dt] = x.fa.v[dt] + (uint32_t)vcur;
    half_step(x, 2 * kb, sa, sb, x.lds + kCur + kHalf * kRowBytes, x.lds, va, qf, st);
    if constexpr (Paged)
        dma_rows_paged(x, vfree, x.vbase, pr, x.voff);
    else
        dma<Paged>(x, vfree, x.vbase, (kb + 3) * kBc, x.voff);
    half_step(x, 2 * kb + 1, sb, sa, x.lds + kNext, x.lds + kHalf * kRowBytes, va, qf, st);
    // vmcnt(2 * kDmaPerTile): only this tile's DMA may still be in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kDmaPerTile));
    __syncthreads();
}

template <bool Paged>
__global__ __launch_bounds__(kThreads, 1) void prefill_causal_kernel(PrefillArgs a, int n_qb,
                                                                     int remap) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
    __shared__ int tbl[Paged ? kPrefillMaxPages : 1];   // paged: the sequence's table row

    const int G = a.H_q / a.H_kv;
    // ---- workgroup -> (q-block, b, h) ----
    int wid = blockIdx.x;
    if (remap) {
        const int x = wid % kXcds, t = wid / kXcds;
        const int j = t % G, u = (t / G) * kXcds + x;
        wid = u * G + j;
    }
    const int j = wid % G;
    int u = wid / G;
    const int hk = u % a.H_kv;
    u /= a.H_kv;
    const int b = u % a.B;
    const int qb = n_qb - 1 - u / a.B;  // heavy (long-prefix) blocks first
    const int h = hk * G + j;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, hf = lane >> 5;
    const int i0 = qb * kBr;
    const int r0 = i0 + w * 32;            // this wave's first query row
    const int row = r0 + r32;              // this lane's query row
    const int last_row = min(i0 + kBr, a.T) - 1;
    // query row i is token qs + i (per sequence when given, clamped so that every key the
    // chunk sees lies in the cache)
    const int qs_raw = a.q_starts ? a.q_starts[b] : a.q_start;
    const int qs = a.q_starts ? min(max(qs_raw, 0), a.q_start_max) : a.q_start;
    // a start outside the table's capacity is clamped (no read past the table), and the
    // sequence's LSE is written as NaN so that the caller can tell
    const bool clamped = qs != qs_raw;

    WaveCtx x;
    x.lds = smem;
    x.kv_row = (size_t)a.H_kv * D;
    if constexpr (Paged) {
        x.kbase = a.k + (size_t)hk * D;          // the pools, head hk
        x.vbase = a.v + (size_t)hk * D;
    } else {
        x.kbase = a.k + ((size_t)b * a.S * a.H_kv + hk) * D;
        x.vbase = a.v + ((size_t)b * a.S * a.H_kv + hk) * D;
    }
    x.tbl = tbl;
    x.page = a.page;
    x.num_pages = a.num_pages;
    // keys past the chunk's last token are never visible: they are not even read, so a
    // cache row after it may hold anything (a zero row times a zero weight adds nothing)
    x.S = qs + a.T;
    x.n_kb = (qs + last_row) / kBc + 1;
    // 32-key steps this wave needs: keys [0, qs + its last real row], the last on its
    // diagonal; the steps that hold a key past the diagonal of its first row are masked
    x.n_sub = r0 < a.T ? (qs + min(r0 + 31, a.T - 1)) / kHalf + 1 : 0;
    x.mask_from = (qs + r0) / kHalf;
    x.w = w;
    x.row = qs + row;
    x.hf = hf;
    // tau * log2(e); a zero scale is replaced by a tiny one so that a masked score
    // (-inf) still scales to -inf: s * 1e-30 is far below fp32 resolution of the result
    x.c = fmaxf(a.scale_log2, 1e-30f);
    {
        const int lr = 4 * w + lane / 16;   // DMA row within each 32-row group
        // (paged: each DMA instruction starts at the wave's own first row)
        const uint32_t rowb = (uint32_t)((Paged ? lane / 16 : lr) * x.kv_row * 2);
        x.koff = rowb + 16u * (uint32_t)((lane & 15) ^ k_swz(lr));
        x.voff = rowb + 16u * (uint32_t)((lane & 15) ^ v_swz(lr));
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8)
            x.fa.k[k8] = (uint32_t)(r32 * kRowBytes + 16 * ((hf * 8 + k8) ^ k_swz(r32)));
        const int vr = 4 * hf + ((lane & 15) >> 2);             // transpose-read row
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within 64 B
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            x.fa.v[dt] = (uint32_t)(vr * kRowBytes + 16 * ((4 * dt + cc) ^ v_swz(vr)) +
                                    8 * (lane & 1));
    }

    // Q^T fragments: column = query row, k-slots (hf, j) <-> d = 64*hf + 8*ks + j
    bf16x8 qf[8];
    {
        const uint16_t *qrow =
            a.q + (((size_t)b * a.T + min(row, a.T - 1)) * a.H_q + h) * D + hf * 64;
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) qf[k8] = as_bf16x8(load16(qrow + k8 * 8));
    }

    RowState st;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][r] = 0.f;
    st.m = neg_inf();
    st.l = 0.f;
    st.lw = 0.f;
    f32x16 sa, sb;

    if constexpr (Paged) {
        // the table entries of the blocks holding keys [0, S), before the first DMA
        const int n = (x.S + a.page - 1) / a.page;
        const int32_t *row = a.block_table + (size_t)b * a.max_blocks;
        for (int i = threadIdx.x; i < n; i += kThreads) tbl[i] = row[i];
        __syncthreads();
    }
    // prologue: K(0..2) and V(0..2) into LDS, then the scores of the first step
    for (int t = 0; t < 3; ++t) dma<Paged>(x, kKBuf + t * kTileBytes, x.kbase, t * kBc, x.koff);
    for (int t = 0; t < 3; ++t) dma<Paged>(x, kVBuf + t * kTileBytes, x.vbase, t * kBc, x.voff);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (x.n_sub > 0) {
        qk_half(sa, smem + kKBuf, x.fa, qf);
        if (x.mask_from == 0) mask_half(sa, 0, x.row, hf);
    }

    int kb = 0;
    for (; kb + 3 < x.n_kb; kb += 4) {
        tile_step<0, Paged>(x, kb, sa, sb, qf, st);
        tile_step<1, Paged>(x, kb + 1, sa, sb, qf, st);
        tile_step<2, Paged>(x, kb + 2, sa, sb, qf, st);
        tile_step<3, Paged>(x, kb + 3, sa, sb, qf, st);
    }
    if (kb < x.n_kb) tile_step<0, Paged>(x, kb, sa, sb, qf, st);
    if (kb + 1 < x.n_kb) tile_step<1, Paged>(x, kb + 1, sa, sb, qf, st);
    if (kb + 2 < x.n_kb) tile_step<2, Paged>(x, kb + 2, sa, sb, qf, st);
    __builtin_amdgcn_s_waitcnt(0);   // no DMA left in flight at exit

    // ---- epilogue: O = O^T / lw -> bf16, LSE = ln2 * (m + log2 l) ----
    // (O leaves through the wave's own 8 KiB of the rings as whole rows; after this barrier
    // every wave's DMA has landed and no wave reads a tile buffer)
    __syncthreads();
    const float l = st.l + __shfl_xor(st.l, 32);
    const float lw = st.lw + __shfl_xor(st.lw, 32);
    static_assert(kWaves * 32 * kRowBytes <= kLdsBytes, "each wave stages its 32 rows");
    store_rows128(st.o, 1.f / lw, smem + w * (32 * kRowBytes),
                  a.o + ((size_t)b * a.T * a.H_q + h) * D, (size_t)a.H_q * D, r0, a.T, lane);
    if (hf == 0 && row < a.T)
        a.lse[((size_t)b * a.H_q + h) * a.T + row] =
            clamped ? __builtin_nanf("") : kLn2 * (st.m + __builtin_log2f(l));
}

}  // namespace

hipError_t launch_prefill_causal(const PrefillArgs &a, hipStream_t stream) {
    if (a.d != D) return hipErrorInvalidValue;
    const int n_qb = (a.T + kBr - 1) / kBr;
    const long units = (long)n_qb * a.B * a.H_kv;
    const int remap = (units % kXcds) == 0;
    const long blocks = units * (a.H_q / a.H_kv);
    if (a.block_table)
        hipLaunchKernelGGL(prefill_causal_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, a, n_qb, remap);
    else
        hipLaunchKernelGGL(prefill_causal_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, a, n_qb, remap);
    return hipGetLastError();
}

}  // namespace gqa
