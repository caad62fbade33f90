/*
 * gqa_attn.h -- C ABI of libgqa_attn.so: grouped-query fused attention on
 * AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The library computes attention of post-RoPE queries against a read-only
 * K/V cache, in the form the pages state it: the attention call sits between
 * the QKV/RoPE/cache-append kernel upstream and the output projection
 * downstream, reads Q, the K cache and the V cache, and writes O; it neither
 * rotates nor writes the cache, and the score matrix S and probabilities P are
 * never produced (ADR-0060 "AHBM GQA Fused Attention", section 0.5: position
 * in the decoder layer, preconditions, launch inputs and outputs).  Query head
 * h reads KV head floor(h / G), G = H_q / H_kv, and H_kv must divide H_q
 * ("Attention Kernel lineage" (V07), section 14).
 *
 * Every call also returns the log-sum-exp of each query row's scores,
 * LSE = m + ln(l) in natural-log units of the scaled logits (V07, section 2:
 * LSE is kept per row instead of S).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major (last index fastest), no padding.
 * - bf16 tensors are passed as `const void*` / `void*` device pointers to
 *   IEEE bfloat16 values; they must be 16-byte aligned.  fp32 and int32
 *   arrays must be 4-byte aligned; the decode workspace 256-byte aligned.
 * - All device pointers are allocated and owned by the caller.  The library
 *   never allocates, frees or synchronises; inputs are read-only; outputs are
 *   fully overwritten.
 * - `stream` is a hipStream_t (NULL = the default stream).  A call returns
 *   after enqueueing its kernels; GQA_OK means the launches were accepted.
 * - Errors are status codes; nothing aborts and no exception crosses the ABI.
 *   All argument checks run on the host before any launch, so a bad shape
 *   fails at the call.  gqa_last_error() gives a one-line explanation of the
 *   most recent failure on the calling thread.
 * - softmax_scale is tau in s = tau * q.k (normally 1/sqrt(d)); any finite
 *   value >= 0 is accepted.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    GQA_ERR_BAD_SHAPE = 2,    /* a size is <= 0, H_kv does not divide H_q, or an index overflows */
    GQA_ERR_UNSUPPORTED = 3,  /* head size (or group size) this build has no kernel for */
    GQA_ERR_SPLITS = 4,       /* num_splits / max_splits out of range */
    GQA_ERR_WORKSPACE = 5,    /* workspace missing, too small or misaligned */
    GQA_ERR_ALIGNMENT = 6,    /* a tensor pointer is not aligned as stated above */
    GQA_ERR_SCALE = 7,        /* softmax_scale is negative, NaN or infinite */
    GQA_ERR_HIP = 8           /* the HIP runtime rejected a launch */
} gqa_status_t;

/* Name of a status code ("GQA_OK", ...); never NULL. */
const char *gqa_status_string(int status);

/* Explanation of the most recent failing call on this thread ("" if none). */
const char *gqa_last_error(void);

/* Library version string. */
const char *gqa_version(void);

/*
 * gqa_device_info -- what the roofline figures are computed from: the number of
 * compute units, the peak engine clock (kHz) and the architecture name of HIP
 * device `device` (the bf16 dense matrix-core peak of a CDNA4 part is
 * compute_units * 4096 FLOP per clock).  Any output pointer may be NULL; `arch`
 * receives at most arch_len bytes, NUL-terminated.  Returns GQA_ERR_BAD_SHAPE for
 * a device index out of range, GQA_ERR_HIP if the runtime fails.
 */
int gqa_device_info(int device, int *compute_units, int *clock_khz, char *arch,
                    size_t arch_len);

/*
 * gqa_stream_read -- the decode's bandwidth ceiling on this device: one launch of
 * a plain streaming-read kernel (one workgroup of 512 threads per compute unit,
 * eight 16-byte loads in flight per thread) over `bytes` bytes of device memory,
 * read once each, as the decode sweep reads each cached K/V byte once (V07,
 * section 14: decode is bound by the K/V bytes read).  Nothing is computed from
 * the data; it is a calibration, timed by the caller.
 *
 *   buf    device memory, 16-byte aligned, read-only; bytes a positive multiple of 16
 *   sink   gqa_stream_read_sink_bytes() bytes of device memory, 4-byte aligned; a
 *          word of it is written only if a workgroup's checksum of the data
 *          happens to equal a fixed constant (which keeps the loads)
 */
size_t gqa_stream_read_sink_bytes(void);
int gqa_stream_read(const void *buf, size_t bytes, void *sink, void *stream);

/*
 * gqa_mfma_rate -- the prefill's matrix-core ceiling on this device for given operand
 * data (V07, section 19: prefill is bound by its matrix products): one launch of a
 * kernel (one workgroup of 512 threads per compute unit) in which every wave runs
 * `iters` rounds of 16 independent bf16 32x32x16 matrix products on 16 operand
 * fragments it loads once from `ops` -- thread t takes the 16-byte words
 * (16 t + i) mod (bytes / 16), i = 0..15 -- and does nothing else.  The rate depends on
 * the operand bits as well as on the instructions (under sustained load the engine
 * clock falls with the switching of random mantissas), so the caller passes data drawn
 * like the prefill's inputs and times the launch.  *flop_out, if flop_out is not NULL,
 * receives the launch's FLOP count.
 *
 *   ops    device memory, 16-byte aligned, read-only; bytes a multiple of 16, >= 256
 *   iters  rounds per wave, 1 .. 1048576
 *   sink   gqa_mfma_rate_sink_bytes() bytes of device memory, 4-byte aligned: thread t
 *          writes the sum of its accumulators (a float) at word t
 */
size_t gqa_mfma_rate_sink_bytes(void);
int gqa_mfma_rate(const void *ops, size_t bytes, int iters, void *sink, double *flop_out,
                  void *stream);

/*
 * Split-KV plan of a decode launch (V07, section 17, split-K decode: the key
 * axis is cut into partitions whose partial states a second stage merges;
 * ADR-0060, section 4: the partial states are combined in two levels).
 *
 * Each sequence's keys [0, seqlen) are cut into 16-key tiles; the tiles of all
 * sequences of the batch, in order (sequence 0's first), are cut into
 * `partitions` equal contiguous ranges, and one workgroup sweeps each range for
 * a group of up to 8 KV heads.  Every time a range leaves a sequence it yields
 * that sequence's partial state, so a sequence gets one state per range that
 * touches it, however ragged the lengths; the merge combines them (the merge is
 * associative: V07, section 3).  partitions = max(num_splits, the number that
 * fills the device: 256 workgroups in total); num_splits = 0 lets the library
 * choose.  A launch whose batch has fewer tiles than that uses one partition
 * per tile.  Partition x and sequence b share state slot x + b, so there are
 * `states` = partitions + B - 1 slots per query head.
 *
 * Outputs (any may be NULL): *partitions_out, *states_out, *workspace_bytes_out
 * (decode workspace the launch needs).
 *
 * Supported: d in {32, 64, 128}; any G = H_q / H_kv (groups above 16 query
 * heads run as several workgroups per KV head); 1 <= B <= 8192;
 * B * ceil(S_max / 16) < 2^31; 0 <= num_splits <= 65535.
 */
int gqa_decode_plan(int B, int H_q, int H_kv, int d, int S_max, int num_splits,
                    int *partitions_out, int *states_out, size_t *workspace_bytes_out);

/*
 * gqa_attn_decode -- one query token per sequence against its KV cache.
 *
 * The G query heads of a KV head are folded into the rows of one matrix
 * product so each K/V tile is read from HBM once for all of them (ADR-0060,
 * TL;DR and section 5.2: M-fold; V07, section 14, GQA kernel layout).  Each
 * partition of the split plan (see gqa_decode_plan) runs an online-softmax
 * sweep (V07, section 2: running (m, l, O) update; section 7: deferred
 * division), then a separate merge kernel combines each sequence's partial
 * states (V07, section 3 merge formula; section 17, second stage of split-K
 * decode).
 * There is no causal mask: the query sees every cached key [0, seqlen)
 * (ADR-0060, section 5.2).
 *
 *   q        [B, H_q, d]        bf16, device, read-only
 *   k_cache  [B, S_max, H_kv, d] bf16, device, read-only (batch stride S_max*H_kv*d)
 *   v_cache  [B, S_max, H_kv, d] bf16, device, read-only
 *   seqlens  [B] int32, device, or NULL (= every sequence has S_max keys).
 *            Rows at or past seqlens[b] are never read.  Values outside
 *            [0, S_max] are clamped into it on the device; seqlens[b] = 0
 *            gives O = 0 and LSE = -inf for that sequence.
 *   o        [B, H_q, d]        bf16, device, written (RNE from fp32)
 *   lse      [B, H_q]           fp32, device, written (natural log)
 *   workspace / workspace_bytes: device scratch of at least the size
 *            gqa_decode_plan reports for the same arguments (256-byte aligned).
 *            Layout, with N = `states` slots per query head, each region starting
 *            at a 256-byte boundary: seg [B][2] int32 (first slot and number of
 *            slots of each sequence's states), then m2 [N][H_q] fp32 (running max,
 *            log2 units), l [N][H_q] fp32, O [N][H_q][d] bf16 (unnormalised,
 *            rounded to nearest even when stored).
 *            Sequence b's states are slots seg[b][0] .. seg[b][0] + seg[b][1] - 1;
 *            other slots are not written.  A state is defined up to a common
 *            shift of its (m2, l, O).
 *
 * Calls that share a workspace on overlapping streams race.
 */
int gqa_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *seqlens, void *o, float *lse,
                    int B, int H_q, int H_kv, int d, int S_max,
                    float softmax_scale, int num_splits,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_attn_decode_noalloc -- gqa_attn_decode for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): the same split plan, kernels and results,
 * with the workspace taken from a device array of the library itself instead of
 * a caller buffer.  Nothing is allocated or freed by this call.
 *
 * Every GPU the library runs on holds one such array of
 * gqa_decode_noalloc_max_workspace() bytes (16 MiB) until the process ends; the
 * first call on a device looks its address up.  A decode whose plan
 * (gqa_decode_plan) needs more workspace is rejected with GQA_ERR_WORKSPACE.
 * All calls on one GPU share its array, so calls that overlap on one GPU (on
 * different streams, or from different threads) race; calls ordered on one
 * stream do not.  Arguments and outputs as gqa_attn_decode.
 */
int gqa_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seqlens, void *o, float *lse, int B, int H_q, int H_kv,
                            int d, int S_max, float softmax_scale, int num_splits, void *stream);
size_t gqa_decode_noalloc_max_workspace(void);

/*
 * The two stages of gqa_attn_decode as separate calls, with the same
 * arguments and workspace layout (V07, section 17: stage 1 writes the partial
 * (m, l, O) of every partition, stage 2 merges them).  gqa_decode_partials
 * runs the split-KV sweep and fills the workspace; gqa_decode_combine runs the
 * merge kernel on it (the workspace carries each sequence's slot range, so the
 * merge needs no lengths).  Calling them in this order on one stream is exactly
 * gqa_attn_decode.
 */
int gqa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seqlens,
                        int B, int H_q, int H_kv, int d, int S_max,
                        float softmax_scale, int num_splits,
                        void *workspace, size_t workspace_bytes, void *stream);

int gqa_decode_combine(void *o, float *lse,
                       int B, int H_q, int H_kv, int d, int S_max, int num_splits,
                       const void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_attn_decode_paged -- gqa_attn_decode over a paged KV cache.
 *
 * The cache lives in fixed-size pages of page_size tokens drawn from a pool,
 * and each sequence lists its pages in a block table: token t of sequence b is
 * row t % page_size of page block_table[b][t / page_size] ("Attention Kernel
 * lineage" (V07), section 16: block pool, block table and the logical-token-to-
 * page map; section 17: paged decode, split-K over the key axis with a second
 * merge stage).  Everything else -- the M-fold of the query rows, the split
 * plan, the merge, the outputs -- is that of gqa_attn_decode_tokens (T_q query
 * tokens per sequence, the last T_q positions; T_q = 1 is gqa_attn_decode), with
 * S_max = max_blocks * page_size; its workspace is sized by
 * gqa_decode_tokens_plan (T_q = 1: gqa_decode_plan).
 *
 *   q           [B, T_q, H_q, d]                   bf16, device, read-only
 *   k_pool      [num_pages, page_size, H_kv, d]    bf16, device, read-only
 *   v_pool      [num_pages, page_size, H_kv, d]    bf16, device, read-only
 *               (K and V are two pools with one page numbering; a page's K rows
 *               and V rows sit at the same page index of each)
 *   block_table [B, max_blocks] int32, device, read-only.  Only the entries of
 *               blocks that hold live tokens (block < ceil(seqlens[b] / page_size))
 *               are read; the rest may hold anything.  A live entry outside
 *               [0, num_pages) is not dereferenced: its keys read as zeros (the
 *               result for that sequence is then meaningless, but nothing faults).
 *               Pages may be shared between sequences.
 *   seqlens     [B] int32, device, or NULL (= max_blocks * page_size tokens each),
 *               clamped to [0, max_blocks * page_size] on the device.
 *   o, lse      [B, T_q, H_q, d] bf16 and [B, H_q, T_q] fp32, as
 *               gqa_attn_decode_tokens (for T_q = 1 the layouts of gqa_attn_decode).
 *   page_size   tokens per page: a multiple of 16 in [16, 65536].
 *   num_pages, max_blocks: pool size and table width; num_pages * page_size and
 *               max_blocks * page_size must be below 2^31.
 *   workspace   sized by gqa_decode_tokens_plan with S_max = max_blocks * page_size.
 *
 * Calls that share a workspace on overlapping streams race.
 */
int gqa_attn_decode_paged(const void *q, const void *k_pool, const void *v_pool,
                          const int32_t *block_table, const int32_t *seqlens, void *o, float *lse,
                          int B, int T_q, int H_q, int H_kv, int d, int page_size, int num_pages,
                          int max_blocks, float softmax_scale, int num_splits,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_attn_decode_tokens -- decode of T_q query tokens per sequence (a short
 * chunk: speculative decoding, small chunked prefill) against its KV cache.
 *
 * The T_q tokens of sequence b are the last T_q of its seqlens[b] cached keys:
 * token i sits at position seqlens[b] - T_q + i and sees keys j <= that
 * position (causal among the new tokens).  The G query heads' T_q tokens are
 * folded into the rows of one matrix product, G * T_q rows per KV head, so each
 * K/V tile is read once for all of them (ADR-0060, section 5.2: Q [G, T_q, d]
 * reshaped to [G * T_q, d] with the KV tile shared by every row; section 0.5.2:
 * T_q is the width of the launch's query block).  Groups of more than 16 rows
 * run as several workgroups per KV head.  Otherwise as gqa_attn_decode, which
 * is the T_q = 1 case.
 *
 *   q        [B, T_q, H_q, d]    bf16, device, read-only
 *   k_cache, v_cache, seqlens: as gqa_attn_decode; a token whose position is
 *            negative (seqlens[b] < T_q) sees no key: O = 0, LSE = -inf.
 *   o        [B, T_q, H_q, d]    bf16, device, written
 *   lse      [B, H_q, T_q]       fp32, device, written (natural log)
 *   workspace: at least the size gqa_decode_tokens_plan reports for the same
 *            arguments; layout as gqa_attn_decode with H_q * T_q rows per slot
 *            (row h * T_q + i).
 *
 * Supported: 1 <= T_q <= 16 (longer chunks: gqa_attn_prefill_chunk); the rest
 * as gqa_attn_decode.
 */
int gqa_decode_tokens_plan(int B, int T_q, int H_q, int H_kv, int d, int S_max, int num_splits,
                           int *partitions_out, int *states_out, size_t *workspace_bytes_out);

int gqa_attn_decode_tokens(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seqlens, void *o, float *lse, int B, int T_q, int H_q,
                           int H_kv, int d, int S_max, float softmax_scale, int num_splits,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_lse_merge -- merge caller-provided partial states (V07, section 3:
 * M = max m_p, a_p = 2^(m_p - M), L = sum a_p l_p, O = sum a_p O_p / L;
 * section 17, second stage).  Partial maxima are in log2 units of the scaled
 * logits (m2 = m * log2(e)), so LSE = ln(2) * (M + log2(L)).  A partial with
 * m2 = -inf is empty and contributes nothing; a row whose partials are all
 * empty gets O = 0 and LSE = -inf.
 *
 *   part_m2  [B, H_q, max_splits] fp32, device, read-only
 *   part_l   [B, H_q, max_splits] fp32, device, read-only (l >= 0)
 *   part_o   [B, H_q, max_splits, d] fp32, device, read-only (unnormalised O),
 *            16-byte aligned
 *   split_counts [B] int32, device, or NULL: partials [0, split_counts[b]) of
 *            sequence b are merged (clamped to [0, max_splits]); NULL = all.
 *   o        [B, H_q, d] bf16, device, written
 *   lse      [B, H_q]    fp32, device, written
 *
 * Supported: d in {32, 64, 128}; 1 <= max_splits <= 65535.
 */
int gqa_lse_merge(const float *part_m2, const float *part_l, const float *part_o,
                  const int32_t *split_counts, int max_splits,
                  void *o, float *lse, int B, int H_q, int d, void *stream);

/*
 * gqa_attn_prefill_causal -- causal self-attention over a whole prompt
 * (T_q = S_kv = S): query i sees keys j <= i (V07, section 12).
 *
 * FlashAttention-2 style: each workgroup keeps one block of query rows and its
 * (m, l, O) state on chip and streams K/V tiles past it, with P.V fused and the
 * score matrix never written (V07, sections 4, 7 and 8); tiles wholly above
 * the diagonal are skipped and only diagonal tiles are masked (V07, section
 * 12: block classification).
 *
 *   q   [B, S, H_q, d]  bf16, device, read-only
 *   k   [B, S, H_kv, d] bf16, device, read-only
 *   v   [B, S, H_kv, d] bf16, device, read-only
 *   o   [B, S, H_q, d]  bf16, device, written (RNE from fp32)
 *   lse [B, H_q, S]     fp32, device, written (natural log)
 *
 * Supported: d = 128.
 */
int gqa_attn_prefill_causal(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int S, int H_q, int H_kv, int d,
                            float softmax_scale, void *stream);

/*
 * gqa_attn_prefill_chunk -- causal attention of a chunk of a sequence against
 * its KV cache: the T_q query rows are the tokens q_start .. q_start + T_q - 1,
 * and query row i sees keys j <= q_start + i (ADR-0060, section 0.5.2: the
 * launch carries the query block's q_start and T_q; section 5.4: each KV tile is
 * wholly past, wholly future or partial for the query block; V07, section 12:
 * causal mask and block classification).  With the chunk at the end of the
 * cache (q_start = S_kv - T_q) this is the bottom-right aligned causal mask of
 * chunked prefill; q_start = 0, T_q = S_kv is gqa_attn_prefill_causal.  Same
 * kernel, tiling and outputs as gqa_attn_prefill_causal.
 *
 *   q        [B, T_q, H_q, d]   bf16, device, read-only
 *   k_cache  [B, S_kv, H_kv, d] bf16, device, read-only (batch stride S_kv*H_kv*d);
 *            rows at or past q_start + T_q are never read and may hold anything
 *   v_cache  [B, S_kv, H_kv, d] bf16, device, read-only (same)
 *   o        [B, T_q, H_q, d]   bf16, device, written (RNE from fp32)
 *   lse      [B, H_q, T_q]      fp32, device, written (natural log)
 *
 * Requires T_q >= 1 and 0 <= q_start <= S_kv - T_q.  Supported: d = 128.
 */
int gqa_attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache, void *o,
                           float *lse, int B, int T_q, int q_start, int S_kv, int H_q, int H_kv,
                           int d, float softmax_scale, void *stream);

/*
 * gqa_attn_prefill_chunk_paged -- gqa_attn_prefill_chunk over a paged KV cache:
 * key t of sequence b is row t % page_size of page block_table[b][t / page_size]
 * of the pools (V07, section 16: block pool, block table, logical-token-to-page
 * map; section 17: the attention kernel reads the cache through the table).  The
 * chunk's T_q query rows are the tokens q_start .. q_start + T_q - 1 of every
 * sequence of the batch and see keys j <= q_start + i, so the keys read are
 * [0, q_start + T_q) of each sequence.  The sequence's table row is staged on
 * chip and each K/V tile is fetched page by page; the results equal those of
 * gqa_attn_prefill_chunk on the gathered cache bit for bit.
 *
 *   q           [B, T_q, H_q, d]                   bf16, device, read-only
 *   k_pool      [num_pages, page_size, H_kv, d]    bf16, device, read-only
 *   v_pool      [num_pages, page_size, H_kv, d]    bf16, device, read-only (one page
 *               numbering with k_pool)
 *   block_table [B, max_blocks] int32, device, read-only; only the entries of blocks
 *               holding keys [0, q_start + T_q) are read.  An entry outside
 *               [0, num_pages) is not dereferenced: its keys read as zeros.  Pool
 *               rows of those blocks at or past q_start + T_q are never read.
 *   q_starts    [B] int32, device, or NULL (= q_start for every sequence): sequence b's
 *               chunk starts at q_starts[b], each sequence at its own position.  A
 *               value outside [0, min(max_blocks, 8192) * page_size - T_q] is clamped
 *               on the device to that range (so no table entry past the row is read),
 *               and that sequence's LSE rows are written as NaN to flag it; its O is
 *               the clamped window's.  (The host checks below apply to q_start only.)
 *   o, lse      [B, T_q, H_q, d] bf16, [B, H_q, T_q] fp32, device, written
 *
 * Requires T_q >= 1, q_start >= 0, ceil((q_start + T_q) / page_size) <= max_blocks
 * and <= 8192 (GQA_ERR_UNSUPPORTED past it: use larger pages); page_size a multiple
 * of 16 in [16, 65536].  Supported: d = 128.
 */
int gqa_attn_prefill_chunk_paged(const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *block_table, const int32_t *q_starts, void *o,
                                 float *lse, int B, int T_q, int q_start, int H_q, int H_kv, int d,
                                 int page_size, int num_pages, int max_blocks,
                                 float softmax_scale, void *stream);

/*
 * FP8 (E4M3) paged KV cache (V07, section 17.7: a per-token scale kept with each
 * page, its page_size scalars appended after the page's rows, dequantisation fused
 * into the load; section 9.5: E4M3 values, fp32 accumulation).  A pool is an array
 * of num_pages pages of gqa_fp8_page_bytes(page_size, H_kv, d) bytes each:
 *
 *   bytes [0, page_size*H_kv*d)           E4M3 codes, [page_size][H_kv][d]
 *   bytes [page_size*H_kv*d, +4*page_size) fp32 scales, one per page row (token)
 *
 * (K and V are two such pools with one page numbering.)  A token's row holds
 * code(x) with x = value(code) * scale.  E4M3 is the OCP 8-bit floating-point
 * format: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
 * subnormals m * 2^-9; 0x7F and 0xFF are NaN; the largest finite value is 448.
 */

/* Bytes of one FP8 page (0 for non-positive sizes). */
size_t gqa_fp8_page_bytes(int page_size, int H_kv, int d);

/*
 * gqa_kv_quantize_fp8 -- write a bf16 cache into the pages of an FP8 pool (the
 * cache-writing step upstream of attention): token t < seqlens[b] of sequence b
 * (NULL seqlens: every t < S_max) is stored in row t % page_size of page
 * block_table[b][t / page_size] as E4M3 codes of its H_kv * d values with one
 * scale 2^e, e the smallest integer with max |x| <= 448 * 2^e (clamped to
 * [-126, 127]; an all-zero row takes -126); each code is the E4M3 value nearest
 * to x * 2^-e, ties to even.  A power-of-two scale makes every dequantised value
 * exactly a bfloat16.  Slots no live token maps to, and tokens whose table entry
 * is outside [0, num_pages), are not written.
 *
 *   x            [B, S_max, H_kv, d] bf16, device, read-only
 *   seqlens      [B] int32, device, or NULL
 *   block_table  [B, max_blocks] int32, device, read-only (max_blocks*page_size >= S_max)
 *   pool         num_pages * gqa_fp8_page_bytes(...) bytes, device, 16-byte aligned, written
 *
 * Supported: d a multiple of 8.
 */
int gqa_kv_quantize_fp8(const void *x, const int32_t *seqlens, const int32_t *block_table,
                        void *pool, int B, int S_max, int H_kv, int d, int page_size,
                        int num_pages, int max_blocks, void *stream);

/*
 * gqa_kv_dequantize_fp8 -- the inverse of gqa_kv_quantize_fp8: token t < seqlens[b]
 * of sequence b is read from row t % page_size of page block_table[b][t / page_size]
 * of an FP8 pool and written to x as bf16 (code value times the row's scale; with
 * the quantiser's power-of-two scales this is exact, the values the FP8 decode
 * attends over).  It lets kernels that read a bf16 cache -- the chunked prefill --
 * run on an FP8 cache (V07, section 17.7: FP8 is the cache's storage format).
 *
 *   pool         num_pages * gqa_fp8_page_bytes(...) bytes, device, 16-byte aligned
 *   seqlens      [B] int32, device, or NULL (= S_max), clamped to [0, S_max]
 *   block_table  [B, max_blocks] int32, device; max_blocks * page_size >= S_max.  A
 *                live entry outside [0, num_pages) gives a zero row.
 *   x            [B, S_max, H_kv, d] bf16, device, 16-byte aligned; rows at or past
 *                seqlens[b] are not written
 *
 * Requires d % 8 == 0 and positive sizes.
 */
int gqa_kv_dequantize_fp8(const void *pool, const int32_t *seqlens, const int32_t *block_table,
                          void *x, int B, int S_max, int H_kv, int d, int page_size, int num_pages,
                          int max_blocks, void *stream);

/*
 * gqa_attn_decode_paged_fp8 -- gqa_attn_decode_paged over FP8 pools: the same
 * arguments, plan, workspace and outputs, with k_pool and v_pool FP8 pools as
 * above.  Codes are converted to bf16 in registers (exactly), each score is
 * scaled by its key's K scale and each weight by its key's V scale as the tiles
 * are consumed, so the cache is read in about half the bytes of bf16 pages.  With
 * the power-of-two scales of gqa_kv_quantize_fp8 the results are those of
 * gqa_attn_decode_paged over bf16 pages holding the dequantised values, bit for bit.
 *
 * Supported: d in {64, 128}; page_size a multiple of 16.
 */
int gqa_attn_decode_paged_fp8(const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *block_table, const int32_t *seqlens, void *o,
                              float *lse, int B, int T_q, int H_q, int H_kv, int d, int page_size,
                              int num_pages, int max_blocks, float softmax_scale, int num_splits,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_prefill_bwd_workspace_bytes -- device workspace (bytes, 256-byte aligned
 * start required) of gqa_attn_prefill_causal_bwd for these sizes, or 0 if the
 * sizes are invalid.  It holds each row's statistics (its LSE in log2 units and
 * D_i = dO_i . O_i): 8 bytes per query row and head, B * H_q * ceil(S/64) * 512.
 */
size_t gqa_prefill_bwd_workspace_bytes(int B, int S, int H_q, int H_kv, int d);

/*
 * gqa_attn_prefill_causal_bwd -- backward of gqa_attn_prefill_causal: given the
 * forward's inputs, its output O and LSE, and the gradient dO of the output,
 * writes the gradients of q, k and v (V07, section 6.1):
 *   P_ij = exp(tau q_i.k_j - LSE_i) (j <= i),  dP_ij = dO_i . v_j,
 *   D_i = dO_i . O_i (section 6.2),  dS_ij = P_ij (dP_ij - D_i),
 *   dQ_i = tau sum_j dS_ij k_j,  dK_j = tau sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
 * with dK and dV of a KV head summed over its G query heads (section 14).  P is
 * formed again from LSE, never stored (section 6.3).  dQ is accumulated with the
 * query block outer and dK, dV with the key block outer, so no atomics are used
 * (section 8; section 6.5); dK and dV of a KV head are summed over its query heads
 * on chip, in a fixed order, so results are bitwise reproducible.
 *
 *   q, o, d_o  [B, S, H_q, d]  bf16, device, read-only (o: the forward's output)
 *   k, v       [B, S, H_kv, d] bf16, device, read-only
 *   lse        [B, H_q, S]     fp32, device, read-only (the forward's LSE)
 *   dq         [B, S, H_q, d]  bf16, device, written (RNE from fp32)
 *   dk, dv     [B, S, H_kv, d] bf16, device, written (RNE from fp32)
 *   workspace  gqa_prefill_bwd_workspace_bytes(B, S, H_q, H_kv, d) bytes, device,
 *              256-byte aligned; scratch, contents on entry ignored
 *
 * Supported: d = 128.
 */
int gqa_attn_prefill_causal_bwd(const void *q, const void *k, const void *v, const void *o,
                                const float *lse, const void *d_o, void *dq, void *dk, void *dv,
                                int B, int S, int H_q, int H_kv, int d, float softmax_scale,
                                void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
