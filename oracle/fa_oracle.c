/*
 * fa_oracle.c -- plain fp64 CPU attention: TEST INFRASTRUCTURE ONLY.
 *
 * This file is the correctness oracle for the GPU attention library. It is
 * called only from the test suite, from the smoke check and from the CPU
 * baseline leg of the benchmark; the product path never links or calls it.
 * It shares no code, header, table or helper with the GPU kernels.
 *
 * What it computes is the plain definition of exact scaled-dot-product
 * attention, written out with no tiling and no online softmax:
 *   - "FlashAttention" explainer page, section "What it is": scores = Q K^T,
 *     softmax of the scores, weights times V (the three standard steps).
 *   - same page, "Checking correctness": the plain reference computes
 *     scale * Q K^T with scale = d^-1/2 by default, masks future keys for
 *     causal attention, then softmax and the product with V.
 *   - same page, "Step 5": the per-row statistic kept beside O is the log of
 *     the softmax normaliser (LSE).
 *   - same page, glossary: causal attention sees itself and earlier
 *     positions; grouped-query attention shares one K/V head between several
 *     query heads.
 *   - "Flash Attention" skill page, "Workflow 2": window_size=(left, right),
 *     (-1, -1) meaning no window, combinable with causal.
 *   - "The One-Line Change ... Flash Attention 2 in HuggingFace": packed
 *     sequences with cumulative lengths never attend across borders.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes of the repository):
 *   - query head h uses K/V head floor(h / (Hq / Hkv));
 *   - when Sq != Sk, query row i sits at key position i + (Sk - Sq)
 *     ("bottom-right" alignment), so a one-token decode query sees its whole
 *     cache;
 *   - window bounds are inclusive: pos - left <= j <= pos + right, a negative
 *     bound means unbounded on that side;
 *   - LSE is the natural log of sum_j exp(s_ij) over visible keys, where
 *     s_ij = scale * q_i . k_j;
 *   - a row with no visible key has O = 0 and LSE = -inf.
 *
 * Arithmetic: every step in double precision, two passes per row (max, then
 * exp/sum/weighted sum).  The only parallelism is OpenMP over independent
 * rows, which does not change any row's arithmetic.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads used by the row loops below (n < 1 leaves the OpenMP default);
 * returns the number now in effect.  For timing the oracle on one core. */
int fa_oracle_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}

/* Is key j visible from query row i?  Sequence lengths sq (queries) and sk
 * (keys); causal / window flags as described above. */
static int visible(long i, long j, long sq, long sk, int causal, int wl, int wr)
{
    long pos = i + (sk - sq); /* key-axis position of query row i */
    if (j < 0 || j >= sk) return 0;
    if (causal && j > pos) return 0;
    if (wl >= 0 && j < pos - wl) return 0;
    if (wr >= 0 && j > pos + wr) return 0;
    return 1;
}

static double dot(const double* a, const double* b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/* One query row against one key/value head: scores, max, exp, sum, output.
 * scores: caller scratch of length sk. */
static void attend_row(const double* qrow, const double* k, const double* v,
                       long kv_stride, long i, long sq, long sk, int d,
                       int causal, int wl, int wr, double scale,
                       double* orow, double* lse, double* scores)
{
    double m = -INFINITY;
    for (long j = 0; j < sk; ++j) {
        if (!visible(i, j, sq, sk, causal, wl, wr)) continue;
        scores[j] = scale * dot(qrow, k + j * kv_stride, d);
        if (scores[j] > m) m = scores[j];
    }
    for (int t = 0; t < d; ++t) orow[t] = 0.0;
    if (m == -INFINITY) { /* no visible key */
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (long j = 0; j < sk; ++j)
        if (visible(i, j, sq, sk, causal, wl, wr)) l += exp(scores[j] - m);
    for (long j = 0; j < sk; ++j) {
        if (!visible(i, j, sq, sk, causal, wl, wr)) continue;
        double p = exp(scores[j] - m) / l;
        const double* vrow = v + j * kv_stride;
        for (int t = 0; t < d; ++t) orow[t] += p * vrow[t];
    }
    *lse = m + log(l);
}

/* Rows of one (sequence, query head) pair.
 *   q:   n query rows, row r at q + r*q_stride, with query index qi[r] in a
 *        sequence of sq queries;
 *   k,v: sk key/value rows of the matching K/V head, row j at k + j*kv_stride;
 *   out: n rows at out + r*o_stride; lse: n values.
 * Returns 0, or -1 if scratch memory could not be allocated. */
int fa_oracle_rows(const double* q, long q_stride, const int64_t* qi, int n, long sq,
                   const double* k, const double* v, long kv_stride, long sk, int d,
                   int causal, int wl, int wr, double scale,
                   double* out, long o_stride, double* lse)
{
    int err = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(sk > 0 ? sk : 1));
        if (!scores) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int r = 0; r < n; ++r)
                attend_row(q + r * q_stride, k, v, kv_stride, qi[r], sq, sk, d,
                           causal, wl, wr, scale, out + r * o_stride, lse + r, scores);
            free(scores);
        }
    }
    return err;
}

/* Padded batch. q,out: [B,Sq,Hq,d]; k,v: [B,Sk,Hkv,d]; lse: [B,Hq,Sq]. */
int fa_oracle_fwd(const double* q, const double* k, const double* v, double* out, double* lse,
                  int B, int Hq, int Hkv, int Sq, int Sk, int d,
                  int causal, int wl, int wr, double scale)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        if (!scores) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(3) schedule(dynamic, 16)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < Hq; ++h)
                    for (int i = 0; i < Sq; ++i) {
                        int g = h / G;
                        const double* qrow = q + (((long)b * Sq + i) * Hq + h) * d;
                        const double* kb = k + ((long)b * Sk * Hkv + g) * d;
                        const double* vb = v + ((long)b * Sk * Hkv + g) * d;
                        double* orow = out + (((long)b * Sq + i) * Hq + h) * d;
                        double* l = lse + ((long)b * Hq + h) * Sq + i;
                        attend_row(qrow, kb, vb, (long)Hkv * d, i, Sq, Sk, d,
                                   causal, wl, wr, scale, orow, l, scores);
                    }
            free(scores);
        }
    }
    return err;
}

/* Score modifiers.  The "FlashAttention" explainer page, "Variants you may
 * meet": ALiBi-style and relative-position biases add a term to the scores,
 * and soft-capping of the scores needs explicit support in the kernel; the
 * project summary lists ALiBi among the supported features.  The pages give
 * no formulas; the readings used here are those of the fast library's
 * forward arguments (alibi_slopes, softcap):
 *   s_ij = scale * q_i . k_j
 *   s_ij <- cap * tanh(s_ij / cap)                 if cap > 0 (soft-capping)
 *   s_ij <- s_ij - slope_h * |pos_i - j|           (ALiBi, slope of query head h)
 * with pos_i = i + (sk - sq) as for the masks; the softmax, O and LSE then
 * follow the plain definition over the modified scores.  This row routine is
 * a separate copy of attend_row so that the unmodified definition stays
 * exactly as written above. */
static void attend_row_mod(const double* qrow, const double* k, const double* v,
                           long kv_stride, long i, long sq, long sk, int d,
                           int causal, int wl, int wr, double scale, double softcap,
                           double slope, double* orow, double* lse, double* scores)
{
    long pos = i + sk - sq; /* key-axis position of query row i */
    double m = -INFINITY;
    for (long j = 0; j < sk; ++j) {
        if (!visible(i, j, sq, sk, causal, wl, wr)) continue;
        double s = scale * dot(qrow, k + j * kv_stride, d);
        if (softcap > 0) s = softcap * tanh(s / softcap);
        s -= slope * fabs((double)(pos - j));
        scores[j] = s;
        if (s > m) m = s;
    }
    for (int t = 0; t < d; ++t) orow[t] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double sum = 0.0;
    for (long j = 0; j < sk; ++j)
        if (visible(i, j, sq, sk, causal, wl, wr)) sum += exp(scores[j] - m);
    for (long j = 0; j < sk; ++j) {
        if (!visible(i, j, sq, sk, causal, wl, wr)) continue;
        double p = exp(scores[j] - m) / sum;
        for (int t = 0; t < d; ++t) orow[t] += p * v[j * kv_stride + t];
    }
    *lse = m + log(sum);
}

/* Padded batch with score modifiers: as fa_oracle_fwd, plus softcap (0 =
 * off) and alibi ([Hq] slopes, or NULL = no bias). */
int fa_oracle_fwd_mod(const double* q, const double* k, const double* v,
                      double* out, double* lse,
                      int B, int Hq, int Hkv, int Sq, int Sk, int d,
                      int causal, int wl, int wr, double scale,
                      double softcap, const double* alibi)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        if (!scores) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(3) schedule(dynamic, 16)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < Hq; ++h)
                    for (int i = 0; i < Sq; ++i) {
                        int g = h / G;
                        double slope = alibi ? alibi[h] : 0.0;
                        attend_row_mod(q + (((long)b * Sq + i) * Hq + h) * d,
                                       k + ((long)b * Sk * Hkv + g) * d,
                                       v + ((long)b * Sk * Hkv + g) * d, (long)Hkv * d,
                                       i, Sq, Sk, d, causal, wl, wr, scale, softcap, slope,
                                       out + (((long)b * Sq + i) * Hq + h) * d,
                                       lse + ((long)b * Hq + h) * Sq + i, scores);
                    }
            free(scores);
        }
    }
    return err;
}

/* Packed sequences. q,out: [total_q,Hq,d]; k,v: [total_k,Hkv,d];
 * lse: [Hq,total_q]; sequence z owns query rows [cu_q[z], cu_q[z+1]) and
 * key rows [cu_k[z], cu_k[z+1]). */
int fa_oracle_varlen(const double* q, const double* k, const double* v, double* out, double* lse,
                     const int32_t* cu_q, const int32_t* cu_k, int nseq,
                     int Hq, int Hkv, int d, int causal, int wl, int wr, double scale)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    long total_q = cu_q[nseq];
    long max_sk = 1;
    for (int z = 0; z < nseq; ++z)
        if (cu_k[z + 1] - cu_k[z] > max_sk) max_sk = cu_k[z + 1] - cu_k[z];
    int err = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)max_sk);
        if (!scores) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 16)
            for (long t = 0; t < total_q; ++t)
                for (int h = 0; h < Hq; ++h) {
                    int z = 0;
                    while (!(cu_q[z] <= t && t < cu_q[z + 1])) ++z;
                    long sq = cu_q[z + 1] - cu_q[z];
                    long sk = cu_k[z + 1] - cu_k[z];
                    long i = t - cu_q[z];
                    int g = h / G;
                    const double* kb = k + ((long)cu_k[z] * Hkv + g) * d;
                    const double* vb = v + ((long)cu_k[z] * Hkv + g) * d;
                    attend_row(q + (t * Hq + h) * d, kb, vb, (long)Hkv * d, i, sq, sk, d,
                               causal, wl, wr, scale, out + (t * Hq + h) * d,
                               lse + (long)h * total_q + t, scores);
                }
            free(scores);
        }
    }
    return err;
}

/* One-token decode against a KV cache. q,out: [B,1,Hq,d];
 * kc,vc: [B,Sk_cap,Hkv,d]; the first cache_seqlens[b] rows of sequence b are
 * its keys (they include the current token); lse: [B,Hq]. */
int fa_oracle_decode(const double* q, const double* kc, const double* vc,
                     const int32_t* cache_seqlens, double* out, double* lse,
                     int B, int Hq, int Hkv, int Sk_cap, int d,
                     int causal, int wl, int wr, double scale)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(Sk_cap > 0 ? Sk_cap : 1));
        if (!scores) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < Hq; ++h) {
                    long sk = cache_seqlens[b];
                    int g = h / G;
                    const double* kb = kc + ((long)b * Sk_cap * Hkv + g) * d;
                    const double* vb = vc + ((long)b * Sk_cap * Hkv + g) * d;
                    attend_row(q + ((long)b * Hq + h) * d, kb, vb, (long)Hkv * d, 0, 1, sk, d,
                               causal, wl, wr, scale, out + ((long)b * Hq + h) * d,
                               lse + (long)b * Hq + h, scores);
                }
            free(scores);
        }
    }
    return err;
}

/* One-token decode against a paged KV cache, optionally appending the new
 * token's key and value first.
 *
 * The pages say only that the fast library's cached-decode call supports a
 * paged cache (project summary, feature list) and that paged layouts cut
 * wasted cache memory (explainer, advice on generation with a cache).  The
 * readings used here:
 *   - the cache is a pool of num_pages pages of page_size token rows,
 *     k_pages/v_pages: [num_pages, page_size, Hkv, d];
 *   - block_table: [B, max_pages] page indices; token t of sequence b is row
 *     t % page_size of page block_table[b][t / page_size];
 *   - cache_seqlens[b] tokens are in the cache.  Without a new token the
 *     query attends over those keys (as in fa_oracle_decode).  With k_new,
 *     v_new ([B, Hkv, d], one new token per sequence) the new token is first
 *     written at position cache_seqlens[b] (through the block table, into
 *     k_pages/v_pages, which are therefore in/out), then the query attends
 *     over cache_seqlens[b] + 1 keys.
 * Keys are gathered one by one into a plain contiguous buffer and then
 * attended exactly as in the contiguous decode above.
 * Returns 0, -1 (allocation), -2 (head counts) or -3 (a position outside the
 * table or a table entry outside the pool). */
int fa_oracle_decode_paged(const double* q, double* k_pages, double* v_pages,
                           const int32_t* block_table, const int32_t* cache_seqlens,
                           const double* k_new, const double* v_new,
                           double* out, double* lse,
                           int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages,
                           int d, int causal, int wl, int wr, double scale)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    int append = k_new != NULL;
    long cap = (long)max_pages * page_size;
    for (int b = 0; b < B; ++b) {
        long n = (long)cache_seqlens[b] + append;
        if (cache_seqlens[b] < 0 || n > cap) return -3;
        for (long t = 0; t < n; t += page_size) {
            int pg = block_table[(long)b * max_pages + t / page_size];
            if (pg < 0 || pg >= num_pages) return -3;
        }
    }
    /* 1. append: the new row goes to position cache_seqlens[b] */
    if (append) {
        for (int b = 0; b < B; ++b) {
            long t = cache_seqlens[b];
            long pg = block_table[(long)b * max_pages + t / page_size];
            long row = pg * page_size + t % page_size;
            for (int g = 0; g < Hkv; ++g)
                for (int c = 0; c < d; ++c) {
                    k_pages[(row * Hkv + g) * d + c] = k_new[((long)b * Hkv + g) * d + c];
                    v_pages[(row * Hkv + g) * d + c] = v_new[((long)b * Hkv + g) * d + c];
                }
        }
    }
    /* 2. attend over the sequence's keys, gathered page by page */
    int err = 0;
#pragma omp parallel
    {
        size_t rows = (size_t)(cap > 0 ? cap : 1);
        double* scores = (double*)malloc(sizeof(double) * rows);
        double* kseq = (double*)malloc(sizeof(double) * rows * (size_t)d);
        double* vseq = (double*)malloc(sizeof(double) * rows * (size_t)d);
        if (!scores || !kseq || !vseq) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int b = 0; b < B; ++b)
                for (int h = 0; h < Hq; ++h) {
                    long sk = (long)cache_seqlens[b] + append;
                    int g = h / G;
                    for (long t = 0; t < sk; ++t) {
                        long pg = block_table[(long)b * max_pages + t / page_size];
                        long row = pg * page_size + t % page_size;
                        for (int c = 0; c < d; ++c) {
                            kseq[t * d + c] = k_pages[(row * Hkv + g) * d + c];
                            vseq[t * d + c] = v_pages[(row * Hkv + g) * d + c];
                        }
                    }
                    attend_row(q + ((long)b * Hq + h) * d, kseq, vseq, d, 0, 1, sk, d,
                               causal, wl, wr, scale, out + ((long)b * Hq + h) * d,
                               lse + (long)b * Hq + h, scores);
                }
        }
        free(scores);
        free(kseq);
        free(vseq);
    }
    return err;
}

/* Gradients of the padded-batch attention (the training backward).
 *
 * The "FlashAttention" explainer page, "Step 5" and "Backward pass in a bit
 * more detail": the backward needs the gradients with respect to the
 * queries, keys and values; the fused kernel rebuilds the weights from
 * recomputed scores and the saved row statistic.  What those gradients are
 * is fixed by the forward definition alone (O = softmax(S) V with
 * S = scale * Q K^T over the visible keys); this function writes out the
 * chain rule of that definition for one row i, with P the row's softmax
 * weights and dO the incoming gradient of the row's output:
 *     dV_j += P_j dO_i                    dP_j = dO_i . V_j
 *     D_i   = sum_j P_j dP_j              dS_j = P_j (dP_j - D_i)
 *     dQ_i  = scale sum_j dS_j K_j        dK_j += scale dS_j Q_i
 * over visible keys j; dK and dV of a K/V head collect every query head of
 * its group (grouped-query attention).  A row with no visible key
 * contributes nothing and gets dQ_i = 0.  The weights are recomputed here
 * from the scores (two passes: max, then exp and sum), not read from a
 * saved LSE.
 *
 * q, dout, dq: [B,Sq,Hq,d]; k, v, dk, dv: [B,Sk,Hkv,d].  Parallel over
 * (sequence, K/V head) pairs, so each thread owns the dK/dV rows it adds to
 * and every sum runs in a fixed order. */
int fa_oracle_bwd(const double* q, const double* k, const double* v, const double* dout,
                  double* dq, double* dk, double* dv,
                  int B, int Hq, int Hkv, int Sq, int Sk, int d,
                  int causal, int wl, int wr, double scale)
{
    if (Hkv <= 0 || Hq % Hkv != 0) return -2;
    int G = Hq / Hkv;
    long kvs = (long)Hkv * d;   /* token stride of k, v, dk, dv */
    long qs = (long)Hq * d;     /* token stride of q, dout, dq */
    for (long t = 0; t < (long)B * Sk * Hkv * d; ++t) { dk[t] = 0.0; dv[t] = 0.0; }
    int err = 0;
#pragma omp parallel
    {
        size_t n = (size_t)(Sk > 0 ? Sk : 1);
        double* p = (double*)malloc(sizeof(double) * n);
        double* dp = (double*)malloc(sizeof(double) * n);
        if (!p || !dp) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int b = 0; b < B; ++b)
                for (int g = 0; g < Hkv; ++g) {
                    const double* kb = k + ((long)b * Sk * Hkv + g) * d;
                    const double* vb = v + ((long)b * Sk * Hkv + g) * d;
                    double* dkb = dk + ((long)b * Sk * Hkv + g) * d;
                    double* dvb = dv + ((long)b * Sk * Hkv + g) * d;
                    for (int h = g * G; h < (g + 1) * G; ++h)
                        for (long i = 0; i < Sq; ++i) {
                            const double* qrow = q + ((long)b * Sq + i) * qs + (long)h * d;
                            const double* gorow = dout + ((long)b * Sq + i) * qs + (long)h * d;
                            double* dqrow = dq + ((long)b * Sq + i) * qs + (long)h * d;
                            for (int c = 0; c < d; ++c) dqrow[c] = 0.0;
                            double m = -INFINITY;
                            for (long j = 0; j < Sk; ++j) {
                                if (!visible(i, j, Sq, Sk, causal, wl, wr)) continue;
                                p[j] = scale * dot(qrow, kb + j * kvs, d);
                                if (p[j] > m) m = p[j];
                            }
                            if (m == -INFINITY) continue;   /* no visible key */
                            double l = 0.0;
                            for (long j = 0; j < Sk; ++j)
                                if (visible(i, j, Sq, Sk, causal, wl, wr)) l += exp(p[j] - m);
                            double D = 0.0;
                            for (long j = 0; j < Sk; ++j) {
                                if (!visible(i, j, Sq, Sk, causal, wl, wr)) continue;
                                p[j] = exp(p[j] - m) / l;
                                dp[j] = dot(gorow, vb + j * kvs, d);
                                D += p[j] * dp[j];
                            }
                            for (long j = 0; j < Sk; ++j) {
                                if (!visible(i, j, Sq, Sk, causal, wl, wr)) continue;
                                const double ds = p[j] * (dp[j] - D);
                                const double* krow = kb + j * kvs;
                                double* dkrow = dkb + j * kvs;
                                double* dvrow = dvb + j * kvs;
                                for (int c = 0; c < d; ++c) {
                                    dqrow[c] += scale * ds * krow[c];
                                    dkrow[c] += scale * ds * qrow[c];
                                    dvrow[c] += p[j] * gorow[c];
                                }
                            }
                        }
                }
        }
        free(p);
        free(dp);
    }
    return err;
}
