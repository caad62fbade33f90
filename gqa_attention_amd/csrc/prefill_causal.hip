// prefill_causal.hip -- causal GQA prefill (T_q = S_kv = S) on gfx950.
//
// FlashAttention-2 forward ("Attention Kernel lineage" (V07), sections 7-8):
// each workgroup owns one block of 128 query rows of one query head for its
// whole life, keeps the rows' (m, l, O) state in registers, and streams 64-key
// K/V tiles through LDS; the division by l is deferred to the end, and the
// score matrix is never written (section 4).  Causal block classification
// (section 12): a tile wholly above the diagonal is never loaded, a tile wholly
// below needs no mask, and only tiles crossing the diagonal are masked
// element-wise with a select.  The classification is also applied per wave
// (32 rows), so a wave skips tiles that are in its own future.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16): scores are formed
// transposed, S^T = K . Q^T, so each lane owns one query row (lane % 32) and
// holds 32 of that row's 64 scores; the row max and sum need one cross-lane
// step.  P.V is formed as O^T = V^T . P^T, whose B operand is exactly the
// softmax output registers, and whose accumulator keeps one query row per lane,
// so the rescale by alpha is a per-lane scalar.  Q (B operand) stays in
// registers; the K fragments are 16-byte LDS reads; V^T fragments (8 keys of
// one d column) come from the row-major V tile through the LDS transpose read.
//
// Scores are kept in log2 units (s2 = acc * tau * log2(e), one fp32 multiply
// folded into the exponent's FMA; V07 section 2, exp2 trick).
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
constexpr int kBr = 128;          // query rows per workgroup
constexpr int kBc = 64;           // keys per tile
constexpr int kWaves = 4;         // 32 query rows per wave
constexpr int kThreads = kWaves * 64;
constexpr int kPitch = D + 8;     // K tile row pitch in bf16 (272 B): conflict-free 16-byte reads
constexpr int kVPitch = D + 32;   // V tile row pitch in bf16 (288 B): conflict-free transpose reads
constexpr int kLoads = kBc * D * 2 / 16 / kThreads;   // 16-byte loads per thread per tensor
constexpr int kXcds = 8;
constexpr float kSlack = 8.f;     // lazy-rescale slack, log2 units: P <= 2^8 between rescales

static_assert(kLoads == 4, "tile staging assumes 4 loads per thread");

struct Stage {
    u32x4 k[kLoads];
    u32x4 v[kLoads];
};

// row_off[i] = (16i + t/16) * kv_row + 8(t%16) is fixed per thread; only the tile base
// moves.  Keys past the sequence end (ragged last tile) are clamped to the last key.
__device__ __forceinline__ void load_stage(Stage &st, const uint16_t *kbase, const uint16_t *vbase,
                                           size_t kv_row, const uint32_t (&row_off)[kLoads],
                                           int k0, int S) {
    if (k0 + kBc <= S) {
        const size_t tb = (size_t)k0 * kv_row;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            st.k[i] = load16(kbase + tb + row_off[i]);
            st.v[i] = load16(vbase + tb + row_off[i]);
        }
    } else {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int key = min(k0 + i * 16 + t / 16, S - 1);
            const size_t off = (size_t)key * kv_row + (t % 16) * 8;
            st.k[i] = load16(kbase + off);
            st.v[i] = load16(vbase + off);
        }
    }
}

__device__ __forceinline__ void store_stage(const Stage &st, uint16_t *ks, uint16_t *vs) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int row = i * 16 + t / 16, col = (t % 16) * 8;
        *reinterpret_cast<u32x4 *>(ks + row * kPitch + col) = st.k[i];
        *reinterpret_cast<u32x4 *>(vs + row * kVPitch + col) = st.v[i];
    }
}

// One 64-key tile for this wave's 32 query rows: S^T = K.Q^T, online softmax, O^T += V^T.P^T.
// DIAG: the tile crosses the diagonal for some row of the wave, so keys j > i are masked;
// a compile-time flag keeps the mask code out of the (far more common) unmasked tiles.
template <bool DIAG>
__device__ __forceinline__ void attend_tile(const uint16_t *ks, const uint16_t *vs,
                                            const bf16x8 (&qf)[8], f32x16 (&o)[4], float &m,
                                            float &l, float &lw, int k0, int row, int r0, float c, int r32,
                                            int hf, int v_row, int v_col) {
    // ---- S^T = K . Q^T : two 32-key sub-tiles ----
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        const uint16_t *krow = ks + (kt * 32 + r32) * kPitch + hf * 64;
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4 *>(krow + k8 * 8));
            s[kt] = mfma32(kf, qf[k8], s[kt]);
        }
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- online softmax on this lane's row (32 of its 64 scores) ----
    // element (kt, r) is key k0 + 32*kt + 8*(r/4) + 4*hf + r%4
    float mx = neg_inf();
    if constexpr (DIAG) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kt * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
                mx = fmaxf(mx, key <= row ? s[kt][r] : neg_inf());
            }
    } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    }
    // Lazy rescale: the running max m (shared by the row's two lanes) moves only when a
    // score passes it by more than kSlack (log2 units); otherwise p = 2^(s2 - m) <= 2^kSlack
    // and O and l keep their scale, and no cross-lane step is needed.  A common shift
    // cancels in O / l (V07 section 3, shift insertion), so the result is the same; the
    // slack only bounds P and spares the O rescale in almost every tile.  The first tile
    // always moves m (m = -inf).
    if (__any(mx * c > m + kSlack)) {
        mx = wave_max_xor(mx, 32);
        const float m_new = fmaxf(m, mx * c);
        const float alpha = exp2_fast(m - m_new);     // 0 on the first tile
        l *= alpha;
        lw *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m = m_new;
    }
    const float neg_m = -m;

    float p[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = exp2_fast(fmaf(s[kt][r], c, neg_m));
            if constexpr (DIAG) {
                const int key = k0 + kt * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
                e = key <= row ? e : 0.f;
            }
            p[kt][r] = e;
        }

    // P^T as B operand, k-step kk (16 keys): slot j <-> S^T element r = 8*(kk%2) + j of
    // sub-tile kk/2, i.e. key 16*kk + 8*(j/4) + 4*hf + j%4.  Two row sums: l of the fp32
    // P gives the LSE; lw of the bf16-rounded P (the weights the matrix product uses)
    // normalises O, so O is an exact convex combination of those weights.
    bf16x8 pf[4];
    float rs = 0.f, rw = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float *pp = &p[kk >> 1][(kk & 1) * 8];
        const u32x4 w = {pack_bf16x2(pp[0], pp[1]), pack_bf16x2(pp[2], pp[3]),
                         pack_bf16x2(pp[4], pp[5]), pack_bf16x2(pp[6], pp[7])};
#pragma unroll
        for (int i = 0; i < 8; ++i) rs += pp[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) rw = add_bf16_pair(w[i], rw);
        pf[kk] = as_bf16x8(w);
    }
    l += rs;       // this lane's half of the row; the halves are added at the end
    lw += rw;

    // ---- O^T += V^T . P^T ----
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // lanes of each 16-lane group point at rows 16kk + 4hf + (lane%16)/4 (+8 for
            // the second half), columns 32dt + 16((lane/16)%2) + 4(lane%4): the transpose
            // read hands lane l the 4 keys of its slot run at column 32dt + lane%32
            const uint16_t *vp = vs + (16 * kk + v_row) * kVPitch + dt * 32 + v_col;
            const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * kVPitch);
            const u32x4 wv = {lo[0], lo[1], hi[0], hi[1]};
            o[dt] = mfma32(as_bf16x8(wv), pf[kk], o[dt]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

__global__ __launch_bounds__(kThreads, 2) void prefill_causal_kernel(PrefillArgs a, int n_qb,
                                                                     int remap) {
    __shared__ __attribute__((aligned(16))) uint16_t ks_buf[2][kBc * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t vs_buf[2][kBc * kVPitch];

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

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r32 = lane & 31, hf = lane >> 5;
    const int v_row = 4 * hf + ((lane & 15) >> 2);          // transpose-read row offset
    const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int i0 = qb * kBr;
    const int r0 = i0 + w * 32;            // this wave's first query row
    const int row = r0 + r32;              // this lane's query row
    const int last_row = min(i0 + kBr, a.S) - 1;
    const int n_kb = last_row / kBc + 1;
    const bool wave_rows = r0 < a.S;

    const size_t kv_row = (size_t)a.H_kv * D;
    const uint16_t *kbase = a.k + ((size_t)b * a.S * a.H_kv + hk) * D;
    const uint16_t *vbase = a.v + ((size_t)b * a.S * a.H_kv + hk) * D;

    // Q^T fragments: column = query row, k-slots (hf, j) <-> d = 64*hf + 8*ks + j
    bf16x8 qf[8];
    {
        const uint16_t *qrow =
            a.q + (((size_t)b * a.S + min(row, a.S - 1)) * a.H_q + h) * D + hf * 64;
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) qf[k8] = as_bf16x8(load16(qrow + k8 * 8));
    }

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m = neg_inf(), l = 0.f, lw = 0.f;
    const float c = a.scale_log2;

    // K/V tiles go through two LDS buffers: tile kb+1 is stored while tile kb is being
    // computed from the other buffer, and the loads of tile kb+2 are in flight meanwhile,
    // so one barrier per tile separates the writers of a buffer from its readers.
    uint32_t row_off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
        row_off[i] = (uint32_t)((i * 16 + threadIdx.x / 16) * kv_row + (threadIdx.x % 16) * 8);
    Stage stage;
    load_stage(stage, kbase, vbase, kv_row, row_off, 0, a.S);
    store_stage(stage, ks_buf[0], vs_buf[0]);
    if (n_kb > 1) load_stage(stage, kbase, vbase, kv_row, row_off, kBc, a.S);
    __syncthreads();

    for (int kb = 0; kb < n_kb; ++kb) {
        const int k0 = kb * kBc;
        const uint16_t *ks = ks_buf[kb & 1];
        const uint16_t *vs = vs_buf[kb & 1];
        if (wave_rows && k0 <= r0 + 31) {   // else: tile wholly in this wave's future
            if (k0 + kBc - 1 > r0)           // crosses this wave's diagonal
                attend_tile<true>(ks, vs, qf, o, m, l, lw, k0, row, r0, c, r32, hf, v_row, v_col);
            else
                attend_tile<false>(ks, vs, qf, o, m, l, lw, k0, row, r0, c, r32, hf, v_row, v_col);
        }
        if (kb + 1 < n_kb) {
            store_stage(stage, ks_buf[(kb + 1) & 1], vs_buf[(kb + 1) & 1]);
            if (kb + 2 < n_kb) load_stage(stage, kbase, vbase, kv_row, row_off, k0 + 2 * kBc, a.S);
        }
        __syncthreads();
    }
    // ---- epilogue: O = O^T / l -> bf16, LSE = ln2 * (m + log2 l) ----
    l += __shfl_xor(l, 32);
    lw += __shfl_xor(lw, 32);
    if (!wave_rows || row >= a.S) return;
    const float inv = 1.f / lw;
    uint16_t *orow = a.o + (((size_t)b * a.S + row) * a.H_q + h) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d = dt * 32 + rq * 8 + hf * 4;
            const int r = rq * 4;
            *reinterpret_cast<u32x2 *>(orow + d) =
                u32x2{pack_bf16x2(o[dt][r] * inv, o[dt][r + 1] * inv),
                      pack_bf16x2(o[dt][r + 2] * inv, o[dt][r + 3] * inv)};
        }
    if (hf == 0) a.lse[((size_t)b * a.H_q + h) * a.S + row] = kLn2 * (m + __builtin_log2f(l));
}

}  // namespace

hipError_t launch_prefill_causal(const PrefillArgs &a, hipStream_t stream) {
    if (a.d != D) return hipErrorInvalidValue;
    const int n_qb = (a.S + kBr - 1) / kBr;
    const long units = (long)n_qb * a.B * a.H_kv;
    const int remap = (units % kXcds) == 0;
    const long blocks = units * (a.H_q / a.H_kv);
    hipLaunchKernelGGL(prefill_causal_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                       n_qb, remap);
    return hipGetLastError();
}

}  // namespace gqa
