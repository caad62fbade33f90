/*
 * oracle.c -- plain, slow, fp64 CPU reference for grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Its users are the tests, the smoke check and the
 * CPU-baseline leg of the benchmark.  It shares no source, header, table or
 * helper with the HIP library.
 *
 * What it computes is the plain definition of attention, not the tiled
 * algorithm (FlashAttention reaches the same result with the same FLOP:
 * "Attention Kernel lineage" (V07), section 4):
 *
 *   for every query row i of head h, with KV head g = floor(h / G), G = H_q/H_kv
 *   ("Attention Kernel lineage", section 14, group formula):
 *     s_j  = tau * sum_c q[i][c] * k_g[j][c]       for every visible key j
 *     m    = max_j s_j                             (safe softmax pass 1,
 *     l    = sum_j exp(s_j - m)                     pass 2,
 *     p_j  = exp(s_j - m) / l                       pass 3; section 2 step 1)
 *     o[c] = sum_j p_j * v_g[j][c]                 (section 1, O = PV)
 *     lse  = m + ln l                              (section 2, LSE kept per row)
 *
 * Visible keys: decode (one query token) sees keys [0, seqlen); the decode
 * step is a pure read of the cache with no mask but the sequence end (ADR-0060
 * "AHBM GQA Fused Attention", sections 0.5.1 and 5.2).  Causal prefill row i
 * sees keys j <= i (V07 section 12, causal definition).  A prefill chunk is
 * T query rows that are the tokens q_start .. q_start + T - 1 of the sequence
 * (ADR-0060 section 0.5.2: T_q is the chunk width, the launch carries the
 * block's q_start and T_q; section 5.4: the query block [q_start, q_start + T)
 * against the cached keys), so its row i sees keys j <= q_start + i.  Keys at
 * or past q_start + T are never visible.  With the chunk at the end of the
 * cache (q_start = S_kv - T) this is the bottom-right aligned causal mask;
 * q_start = 0, T = S_kv is plain causal prefill.
 *
 * All bf16 inputs are widened exactly to double; every product and sum is in
 * double.  A row with no visible key gives o = 0 and lse = -inf (the identity
 * state (-inf, 0, 0) of the merge, V07 section 3).
 *
 * The partial-state and merge functions restate V07 section 3 (partial
 * definition over a key subset and the combination formula) and section 17
 * (second stage of split-K decode): they let the tests check that merging the
 * states of any partition of the keys gives the unsplit result.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Exact widening of a bfloat16 bit pattern (the high half of an IEEE single). */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One query row against n key/value rows.
 * krow(j) = k + j*kv_stride, vrow(j) = v + j*kv_stride, each d bf16 values.
 * s is caller scratch of n doubles; o receives d doubles. */
static void attend_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       size_t kv_stride, int n, int d, double tau,
                       double *s, double *qd, double *o, double *lse)
{
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (n <= 0) {
        *lse = -INFINITY;
        return;
    }
    for (int c = 0; c < d; ++c) qd[c] = bf16_to_double(q[c]);

    /* the whole score row, materialised */
    for (int j = 0; j < n; ++j) {
        const uint16_t *kj = k + (size_t)j * kv_stride;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qd[c] * bf16_to_double(kj[c]);
        s[j] = tau * dot;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: denominator */
    double l = 0.0;
    for (int j = 0; j < n; ++j) l += exp(s[j] - m);
    /* pass 3: probabilities, then the weighted sum of V */
    for (int j = 0; j < n; ++j) {
        double p = exp(s[j] - m) / l;
        const uint16_t *vj = v + (size_t)j * kv_stride;
        for (int c = 0; c < d; ++c) o[c] += p * bf16_to_double(vj[c]);
    }
    *lse = m + log(l);
}

/* ------------------------------------------------------------------------- */
/* A tiny thread pool over row indices: worker t takes rows t, t+T, t+2T, ... */

typedef void (*row_fn)(void *ctx, long row, double *s, double *qd);

struct pool_arg {
    row_fn fn;
    void *ctx;
    long nrows;
    int tid, nthreads;
    int scratch_n, d;
};

static void *pool_worker(void *p)
{
    struct pool_arg *a = (struct pool_arg *)p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(a->scratch_n > 0 ? a->scratch_n : 1));
    double *qd = (double *)malloc(sizeof(double) * (size_t)a->d);
    if (s && qd)
        for (long r = a->tid; r < a->nrows; r += a->nthreads) a->fn(a->ctx, r, s, qd);
    free(s);
    free(qd);
    return NULL;
}

static int resolve_threads(int nthreads)
{
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run_rows(row_fn fn, void *ctx, long nrows, int nthreads, int scratch_n, int d)
{
    nthreads = resolve_threads(nthreads);
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    struct pool_arg *args = (struct pool_arg *)malloc(sizeof(struct pool_arg) * (size_t)nthreads);
    if (!th || !args) {
        free(th);
        free(args);
        return -1;
    }
    for (int t = 0; t < nthreads; ++t) {
        args[t] = (struct pool_arg){fn, ctx, nrows, t, nthreads, scratch_n, d};
        if (t > 0) pthread_create(&th[t], NULL, pool_worker, &args[t]);
    }
    pool_worker(&args[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(args);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Decode: q [B, H_q, d]; k, v [B, S_max, H_kv, d]; seqlens [B] or NULL.
 * o [B, H_q, d] (double), lse [B, H_q] (double, natural log). */

struct decode_ctx {
    const uint16_t *q, *k, *v;
    const int32_t *seqlens;
    double *o, *lse;
    int B, H_q, H_kv, d, S_max;
    double tau;
};

static void decode_row(void *p, long r, double *s, double *qd)
{
    struct decode_ctx *c = (struct decode_ctx *)p;
    int b = (int)(r / c->H_q), h = (int)(r % c->H_q);
    int G = c->H_q / c->H_kv;
    int g = h / G;
    int n = c->seqlens ? c->seqlens[b] : c->S_max;
    const uint16_t *k0 = c->k + ((size_t)b * c->S_max * c->H_kv + g) * c->d;
    const uint16_t *v0 = c->v + ((size_t)b * c->S_max * c->H_kv + g) * c->d;
    attend_row(c->q + (size_t)r * c->d, k0, v0, (size_t)c->H_kv * c->d, n, c->d, c->tau, s, qd,
               c->o + (size_t)r * c->d, c->lse + r);
}

int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seqlens,
                  double *o, double *lse, int B, int H_q, int H_kv, int d, int S_max,
                  double tau, int nthreads)
{
    if (H_kv <= 0 || H_q % H_kv != 0) return -1;
    if (seqlens)
        for (int b = 0; b < B; ++b)
            if (seqlens[b] < 0 || seqlens[b] > S_max) return -2;
    struct decode_ctx c = {q, k, v, seqlens, o, lse, B, H_q, H_kv, d, S_max, tau};
    return run_rows(decode_row, &c, (long)B * H_q, nthreads, S_max, d);
}

/* ------------------------------------------------------------------------- */
/* Causal prefill of a chunk, on selected rows.
 * q [B, T, H_q, d]; k, v [B, S_kv, H_kv, d]; rows: nrows triples (b, h, i), 0 <= i < T;
 * query row i is token q_start + i, and q_start + T <= S_kv.
 * o [nrows, d] (double), lse [nrows] (double). */

struct prefill_ctx {
    const uint16_t *q, *k, *v;
    const int32_t *rows;
    double *o, *lse;
    int B, T, q_start, S_kv, H_q, H_kv, d;
    double tau;
};

static void prefill_row(void *p, long r, double *s, double *qd)
{
    struct prefill_ctx *c = (struct prefill_ctx *)p;
    int b = c->rows[3 * r], h = c->rows[3 * r + 1], i = c->rows[3 * r + 2];
    int G = c->H_q / c->H_kv;
    int g = h / G;
    const uint16_t *qrow = c->q + (((size_t)b * c->T + i) * c->H_q + h) * c->d;
    const uint16_t *k0 = c->k + ((size_t)b * c->S_kv * c->H_kv + g) * c->d;
    const uint16_t *v0 = c->v + ((size_t)b * c->S_kv * c->H_kv + g) * c->d;
    /* row i is token q_start + i: causal, keys 0 .. q_start + i inclusive */
    int pos = c->q_start + i;
    attend_row(qrow, k0, v0, (size_t)c->H_kv * c->d, pos + 1, c->d, c->tau, s, qd,
               c->o + (size_t)r * c->d, c->lse + r);
}

int oracle_prefill_chunk_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              double *o, double *lse, int B, int T, int q_start, int S_kv,
                              int H_q, int H_kv, int d, double tau, const int32_t *rows,
                              long nrows, int nthreads)
{
    if (H_kv <= 0 || H_q % H_kv != 0) return -1;
    if (T <= 0 || q_start < 0 || q_start > S_kv - T) return -3;
    for (long r = 0; r < nrows; ++r) {
        int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H_q || i < 0 || i >= T) return -2;
    }
    struct prefill_ctx c = {q, k, v, rows, o, lse, B, T, q_start, S_kv, H_q, H_kv, d, tau};
    return run_rows(prefill_row, &c, nrows, nthreads, S_kv, d);
}

/* Whole-prompt causal prefill: the chunk that is the whole sequence (q_start = 0, T = S). */
int oracle_prefill_causal_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               double *o, double *lse, int B, int S, int H_q, int H_kv, int d,
                               double tau, const int32_t *rows, long nrows, int nthreads)
{
    return oracle_prefill_chunk_rows(q, k, v, o, lse, B, S, 0, S, H_q, H_kv, d, tau, rows, nrows,
                                     nthreads);
}

/* ------------------------------------------------------------------------- */
/* Partial state of a decode row over keys [j0, j1) (V07 section 3, partial definition):
 *   m = max s_j,  l = sum exp(s_j - m),  O = sum exp(s_j - m) * v_j   (O not divided by l)
 * The empty range gives the identity (-inf, 0, 0).
 * m, l [B, H_q]; o [B, H_q, d]. */

struct partial_ctx {
    const uint16_t *q, *k, *v;
    double *m, *l, *o;
    int B, H_q, H_kv, d, S_max, j0, j1;
    double tau;
};

static void partial_row(void *p, long r, double *s, double *qd)
{
    struct partial_ctx *c = (struct partial_ctx *)p;
    int b = (int)(r / c->H_q), h = (int)(r % c->H_q);
    int g = h / (c->H_q / c->H_kv);
    int n = c->j1 - c->j0;
    double *o = c->o + (size_t)r * c->d;
    for (int x = 0; x < c->d; ++x) o[x] = 0.0;
    if (n <= 0) {
        c->m[r] = -INFINITY;
        c->l[r] = 0.0;
        return;
    }
    size_t stride = (size_t)c->H_kv * c->d;
    const uint16_t *k0 = c->k + (((size_t)b * c->S_max + c->j0) * c->H_kv + g) * c->d;
    const uint16_t *v0 = c->v + (((size_t)b * c->S_max + c->j0) * c->H_kv + g) * c->d;
    const uint16_t *qr = c->q + (size_t)r * c->d;
    for (int x = 0; x < c->d; ++x) qd[x] = bf16_to_double(qr[x]);
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int x = 0; x < c->d; ++x) dot += qd[x] * bf16_to_double(k0[j * stride + x]);
        s[j] = c->tau * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        double e = exp(s[j] - m);
        l += e;
        for (int x = 0; x < c->d; ++x) o[x] += e * bf16_to_double(v0[j * stride + x]);
    }
    c->m[r] = m;
    c->l[r] = l;
}

int oracle_decode_partial(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          double *m, double *l, double *o, int B, int H_q, int H_kv, int d,
                          int S_max, double tau, int j0, int j1, int nthreads)
{
    if (H_kv <= 0 || H_q % H_kv != 0) return -1;
    if (j0 < 0 || j1 > S_max || j0 > j1) return -2;
    struct partial_ctx c = {q, k, v, m, l, o, B, H_q, H_kv, d, S_max, j0, j1, tau};
    return run_rows(partial_row, &c, (long)B * H_q, nthreads, S_max, d);
}

/* Merge of P partial states per row (V07 section 3 combination formula, applied
 * over all partials at once as in the second stage of split-K decode, section 17):
 *   M = max_p m_p,  a_p = exp(m_p - M),  L = sum a_p l_p,
 *   O = (sum a_p O_p) / L,  lse = M + ln L.
 * A partial with m_p = -inf contributes a_p = 0; all partials empty gives O = 0, lse = -inf.
 * m, l [R, P]; o [R, P, d]; o_out [R, d]; lse_out [R]. */
int oracle_merge_states(const double *m, const double *l, const double *o, long R, int P, int d,
                        double *o_out, double *lse_out)
{
    for (long r = 0; r < R; ++r) {
        const double *mr = m + r * P, *lr = l + r * P, *orow = o + r * (long)P * d;
        double *out = o_out + r * d;
        for (int x = 0; x < d; ++x) out[x] = 0.0;
        double M = -INFINITY;
        for (int p = 0; p < P; ++p)
            if (mr[p] > M) M = mr[p];
        if (M == -INFINITY) {
            lse_out[r] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int p = 0; p < P; ++p) {
            double a = exp(mr[p] - M);
            L += a * lr[p];
            for (int x = 0; x < d; ++x) out[x] += a * orow[(long)p * d + x];
        }
        for (int x = 0; x < d; ++x) out[x] /= L;
        lse_out[r] = M + log(L);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward of whole-prompt causal prefill.
 *
 * Forward (the definition above): s_ij = tau q_i.k_j for j <= i, P_ij = exp(s_ij - LSE_i),
 * O_i = sum_j P_ij v_j.  Given the output gradient dO, the input gradients are
 * ("Attention Kernel lineage" (V07), section 6.1, gradient formulas):
 *   dP_ij = dO_i . v_j           D_i   = sum_j P_ij dP_ij   (the row-wise dot)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = tau sum_j dS_ij k_j  dK_j  = tau sum_i dS_ij q_i  dV_j = sum_i P_ij dO_i
 * with i, j over the causal pairs j <= i.  With grouped heads, K and V of head g are used
 * by the G query heads h with floor(h / G) = g (V07 section 14), so dK and dV of head g
 * add up the contributions of those G heads.
 *
 * Phase 1 (one query row i of head h): the score row, the three-pass softmax, dP_i, D_i
 * and dS_i, then dQ_i; LSE_i and D_i are kept for phase 2.
 * Phase 2 (one key row j of KV head g): for every query row i >= j of the G heads it forms
 * P_ij = exp(s_ij - LSE_i) again and dS_ij from dP_ij and D_i (section 6.4: the backward
 * recomputes P from the row's LSE), and sums dK_j and dV_j.
 * Layouts: q, dO [B, S, H_q, d]; k, v [B, S, H_kv, d] (bf16 bits); dq [B, S, H_q, d],
 * dk, dv [B, S, H_kv, d], lse and D [B, H_q, S] (double). */

struct bwd_rows_ctx {
    const uint16_t *q, *k, *v, *dout;
    const int32_t *rows;
    const double *D_in;
    double *dq, *lse, *D;
    int B, S, H_q, H_kv, d;
    double tau;
};

static void bwd_row(void *p, long r, double *s, double *qd)
{
    struct bwd_rows_ctx *c = (struct bwd_rows_ctx *)p;
    int b = c->rows[3 * r], h = c->rows[3 * r + 1], i = c->rows[3 * r + 2];
    int G = c->H_q / c->H_kv;
    int g = h / G;
    int d = c->d;
    size_t kv_stride = (size_t)c->H_kv * d;
    size_t qoff = (((size_t)b * c->S + i) * c->H_q + h) * d;
    const uint16_t *k0 = c->k + ((size_t)b * c->S * c->H_kv + g) * d;
    const uint16_t *v0 = c->v + ((size_t)b * c->S * c->H_kv + g) * d;
    double *dp = s + c->S;          /* scratch: s[0..S), dp[0..S), dod[0..d) */
    double *dod = s + 2 * (size_t)c->S;
    int n = i + 1;                  /* keys 0 .. i */
    for (int x = 0; x < d; ++x) {
        qd[x] = bf16_to_double(c->q[qoff + x]);
        dod[x] = bf16_to_double(c->dout[qoff + x]);
    }
    for (int j = 0; j < n; ++j) {
        const uint16_t *kj = k0 + (size_t)j * kv_stride;
        const uint16_t *vj = v0 + (size_t)j * kv_stride;
        double dot = 0.0, dpj = 0.0;
        for (int x = 0; x < d; ++x) {
            dot += qd[x] * bf16_to_double(kj[x]);
            dpj += dod[x] * bf16_to_double(vj[x]);
        }
        s[j] = c->tau * dot;
        dp[j] = dpj;
    }
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int j = 0; j < n; ++j) l += exp(s[j] - m);
    for (int j = 0; j < n; ++j) s[j] = exp(s[j] - m) / l;   /* s now holds P_i */
    double D = 0.0;
    for (int j = 0; j < n; ++j) D += s[j] * dp[j];
    if (c->D_in) D = c->D_in[r];   /* D_i = dO_i . O_i of a stored output (section 6.2) */
    double *dq = c->dq + (size_t)r * d;
    for (int x = 0; x < d; ++x) dq[x] = 0.0;
    for (int j = 0; j < n; ++j) {
        double ds = s[j] * (dp[j] - D);
        const uint16_t *kj = k0 + (size_t)j * kv_stride;
        for (int x = 0; x < d; ++x) dq[x] += ds * bf16_to_double(kj[x]);
    }
    for (int x = 0; x < d; ++x) dq[x] *= c->tau;
    c->lse[r] = m + log(l);
    c->D[r] = D;
}

/* Phase 1 on selected rows (b, h, i): dq [nrows, d], lse [nrows], D [nrows].
 * D_in [nrows] or NULL: when given, dS uses D_in[r] in place of the exact row-wise dot --
 * the D_i = dO_i . O_i of section 6.2 taken from a stored (rounded) forward output O,
 * as the method computes it -- and D[r] returns D_in[r]. */
int oracle_prefill_causal_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const uint16_t *dout, const double *D_in, double *dq,
                                   double *lse, double *D, int B, int S, int H_q, int H_kv,
                                   int d, double tau, const int32_t *rows, long nrows,
                                   int nthreads)
{
    if (H_kv <= 0 || H_q % H_kv != 0) return -1;
    for (long r = 0; r < nrows; ++r) {
        int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H_q || i < 0 || i >= S) return -2;
    }
    struct bwd_rows_ctx c = {q, k, v, dout, rows, D_in, dq, lse, D, B, S, H_q, H_kv, d, tau};
    return run_rows(bwd_row, &c, nrows, nthreads, 2 * S + d, d);
}

struct bwd_keys_ctx {
    const uint16_t *q, *k, *v, *dout;
    const double *lse, *D;
    const int32_t *keys;
    double *dk, *dv;
    int B, S, H_q, H_kv, d;
    double tau;
};

static void bwd_key(void *p, long r, double *s, double *kd)
{
    struct bwd_keys_ctx *c = (struct bwd_keys_ctx *)p;
    int b = c->keys[3 * r], g = c->keys[3 * r + 1], j = c->keys[3 * r + 2];
    int G = c->H_q / c->H_kv;
    int d = c->d;
    double *vd = s;                 /* scratch: vd[0..d) */
    size_t koff = (((size_t)b * c->S + j) * c->H_kv + g) * d;
    for (int x = 0; x < d; ++x) {
        kd[x] = bf16_to_double(c->k[koff + x]);
        vd[x] = bf16_to_double(c->v[koff + x]);
    }
    double *dk = c->dk + (size_t)r * d, *dv = c->dv + (size_t)r * d;
    for (int x = 0; x < d; ++x) dk[x] = dv[x] = 0.0;
    for (int h = g * G; h < (g + 1) * G; ++h) {
        const double *lse = c->lse + ((size_t)b * c->H_q + h) * c->S;
        const double *D = c->D + ((size_t)b * c->H_q + h) * c->S;
        for (int i = j; i < c->S; ++i) {   /* query rows that see key j */
            size_t qoff = (((size_t)b * c->S + i) * c->H_q + h) * d;
            double dot = 0.0, dpij = 0.0;
            for (int x = 0; x < d; ++x) {
                dot += bf16_to_double(c->q[qoff + x]) * kd[x];
                dpij += bf16_to_double(c->dout[qoff + x]) * vd[x];
            }
            double pij = exp(c->tau * dot - lse[i]);
            double ds = pij * (dpij - D[i]);
            for (int x = 0; x < d; ++x) {
                dv[x] += pij * bf16_to_double(c->dout[qoff + x]);
                dk[x] += c->tau * ds * bf16_to_double(c->q[qoff + x]);
            }
        }
    }
}

/* Phase 2 on selected key rows (b, g, j), given LSE and D of every row [B, H_q, S] (from
 * phase 1): dk, dv [nkeys, d]. */
int oracle_prefill_causal_bwd_keys(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const uint16_t *dout, const double *lse, const double *D,
                                   double *dk, double *dv, int B, int S, int H_q, int H_kv, int d,
                                   double tau, const int32_t *keys, long nkeys, int nthreads)
{
    if (H_kv <= 0 || H_q % H_kv != 0) return -1;
    for (long r = 0; r < nkeys; ++r) {
        int b = keys[3 * r], g = keys[3 * r + 1], j = keys[3 * r + 2];
        if (b < 0 || b >= B || g < 0 || g >= H_kv || j < 0 || j >= S) return -2;
    }
    struct bwd_keys_ctx c = {q, k, v, dout, lse, D, keys, dk, dv, B, S, H_q, H_kv, d, tau};
    return run_rows(bwd_key, &c, nkeys, nthreads, d, d);
}

/* ------------------------------------------------------------------------- */
/* FP8 KV cache ("Attention Kernel lineage" (V07), section 17.7: a per-token scale kept
 * with each page, the page's B_p scalars appended after its rows, and dequantisation
 * fused into the load; section 9.5: E4M3 values with fp32 accumulation).
 *
 * E4M3 as the OCP 8-bit floating-point specification defines it (its "E4M3" encoding,
 * without infinities): bit 7 is the sign, bits 6..3 a biased exponent (bias 7), bits
 * 2..0 the mantissa.  Exponent field 0 holds zero and the subnormals m * 2^-9; field e > 0
 * holds (1 + m/8) * 2^(e - 7); 0x7F and 0xFF are NaN, so the largest finite value is
 * 0x7E = 1.75 * 2^8 = 448.
 *
 * A token's row (its H_kv * d values of one pool) is quantised with one scale 2^e, e the
 * smallest integer with max |x| <= 448 * 2^e (clamped to [-126, 127]; an all-zero row
 * takes -126), and codes the E4M3 values nearest to x * 2^-e, ties to the even code.
 * The scale is a power of two so that x * 2^-e is exact and code * 2^e is exactly a
 * bfloat16 (4 significant bits), which the tests use. */

double oracle_e4m3_value(int code)
{
    code &= 0xFF;
    int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    if (ex == 15 && man == 7) return NAN;
    double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* The code of the finite E4M3 value nearest to y (ties: the code with an even mantissa);
 * |y| beyond 448 gives +-448, NaN gives 0x7F.  The non-negative finite codes 0x00..0x7E
 * have ascending values, so the two neighbours of |y| are found by bisection. */
int oracle_e4m3_encode(double y)
{
    if (y != y) return 0x7F;
    int sign = signbit(y) ? 0x80 : 0;
    double a = fabs(y);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E;                  /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_value(mid) <= a) lo = mid;
        else hi = mid;
    }
    double dlo = a - oracle_e4m3_value(lo), dhi = oracle_e4m3_value(hi) - a;
    int c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) == 0 ? lo : hi);
    return sign | c;
}

/* The scale exponent of a row whose largest magnitude is amax (see above). */
int oracle_e4m3_scale_exponent(double amax)
{
    if (!(amax > 0.0)) return -126;
    int e = -126;
    while (e < 127 && amax > ldexp(448.0, e)) ++e;
    return e;
}

/* Quantise nrows rows of `width` bf16 values: codes [nrows][width], scales [nrows]. */
void oracle_quantize_fp8_rows(const uint16_t *x, long nrows, int width, uint8_t *codes,
                              float *scales)
{
    for (long r = 0; r < nrows; ++r) {
        const uint16_t *row = x + (size_t)r * width;
        double amax = 0.0;
        for (int i = 0; i < width; ++i) {
            double a = fabs(bf16_to_double(row[i]));
            if (a > amax) amax = a;
        }
        int e = oracle_e4m3_scale_exponent(amax);
        for (int i = 0; i < width; ++i)
            codes[(size_t)r * width + i] = (uint8_t)oracle_e4m3_encode(ldexp(bf16_to_double(row[i]), -e));
        scales[r] = (float)ldexp(1.0, e);
    }
}
