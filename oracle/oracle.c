/*
 * oracle.c -- plain, slow CPU reference for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load
 * or call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP library.
 *
 * Everything is computed in IEEE double from the definitions on the pages, with
 * plain nested loops in the order the definitions state.  The only parallelism
 * is an optional split of independent output rows / sequences over POSIX
 * threads; it does not change any arithmetic inside a row or sequence.
 *
 * Sources (page title, section):
 *   [KV]  "KV Cache + Speculative Decoding" (AI knowledge base)
 *   [SD]  "50 | Speculative Decoding" (Transformer and attention series)
 *   [L10] "Lecture 10 - Inference" (CS336 notes)
 *   [WC]  "Speculative decoding and KV cache optimisation"
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_KV_F32 = 0, OR_KV_BF16 = 1, OR_KV_FP8_E4M3 = 2 };

/* ------------------------------------------------------------------ decoders */

/* bfloat16, from the format definition: 1 sign bit, 8 exponent bits (bias 127),
 * 7 fraction bits; exponent 0 is subnormal, exponent 255 is inf/NaN. */
double oracle_decode_bf16(uint16_t bits)
{
    int s = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double sign = s ? -1.0 : 1.0;
    if (e == 0xFF)
        return m ? NAN : sign * INFINITY;
    if (e == 0)
        return sign * ldexp((double)m / 128.0, -126);
    return sign * ldexp(1.0 + (double)m / 128.0, e - 127);
}

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign bit, 4 exponent bits (bias 7),
 * 3 fraction bits, no infinities, S.1111.111 is NaN, largest finite is 448.
 * The pages store the KV cache in 8-bit float and compute in a wider type
 * ([KV] section 4.5 on KV quantisation; [WC] section 3.5). */
double oracle_decode_e4m3(uint8_t bits)
{
    int s = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double sign = s ? -1.0 : 1.0;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        return sign * ldexp((double)m / 8.0, -6);
    return sign * ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* One cached element as a real number: the stored value, times the per-block
 * scale for 8-bit storage. */
static double kv_elem(const void *cache, int kv_dtype, const float *scale,
                      int64_t blk, int64_t idx)
{
    switch (kv_dtype) {
    case OR_KV_F32:
        return (double)((const float *)cache)[idx];
    case OR_KV_BF16:
        return oracle_decode_bf16(((const uint16_t *)cache)[idx]);
    default:
        return oracle_decode_e4m3(((const uint8_t *)cache)[idx]) * (double)scale[blk];
    }
}

/* ----------------------------------------------------------------- attention */

typedef struct {
    const float *q;
    const void *k_cache, *v_cache;
    const float *k_scale, *v_scale;
    const int32_t *block_table, *context_lens;
    int B, T, Hq, Hkv, d, block_size, max_blocks, kv_dtype;
    double sm_scale;
    const int64_t *rows;
    int64_t nrows;
    double *out;
    double *scratch; /* per thread: score[max_blocks*block_size] */
    const uint32_t *tree_mask; /* [B][T] ancestor sets, or NULL for the chain */
} attn_job;

/*
 * One output row (b, t, h) of verify attention, from the definition.
 *
 * The verify forward feeds [last token, x_1 .. x_K] (T = K+1 rows) after their
 * K/V were appended to the cache, so the cache holds L_b positions including
 * the T new ones and row t sits at position L_b - T + t; it may attend to
 * positions 0 .. L_b - T + t ([KV] 6.1 and 6.3: concatenate, then the causal
 * mask tril with diagonal L_total - L_new; [KV] 7.6 step 2).
 * Query head h reads KV head floor(h / G), G = Hq / Hkv ([KV] 6.3,
 * repeat_interleave over the head axis).
 * Logical position p lives in physical block block_table[b][p / 16], slot
 * p mod 16 ([KV] 5.2-5.3; [L10] 9.2).  Cache layout [block][slot][kv head][d].
 * Scores are q.k * sm_scale (sm_scale = 1/sqrt(d) in [KV] 6.1), softmax over
 * the visible positions, output = softmax-weighted sum of values.
 */
static void attn_one_row(const attn_job *J, int64_t row, double *score, double *o)
{
    const int T = J->T, Hq = J->Hq, Hkv = J->Hkv, d = J->d, bs = J->block_size;
    const int64_t b = row / ((int64_t)T * Hq);
    const int t = (int)((row / Hq) % T);
    const int h = (int)(row % Hq);
    const int G = Hq / Hkv;
    const int g = h / G;
    const int64_t L = J->context_lens[b];
    const int64_t n_vis = L - T + 1 + t;
    const float *qrow = J->q + row * d;
    /* tree verification: row t sees the prefix and the tree nodes j with bit
     * j of its ancestor set (itself included) */
    const uint32_t anc = J->tree_mask ? J->tree_mask[b * T + t] : 0u;

    for (int c = 0; c < d; ++c)
        o[c] = 0.0;
    if (n_vis <= 0) {
        for (int c = 0; c < d; ++c)
            o[c] = NAN;
        return;
    }

    double smax = -INFINITY;
    for (int64_t p = 0; p < n_vis; ++p) {
        if (J->tree_mask && p >= L - T && !((anc >> (p - (L - T))) & 1u)) {
            score[p] = -INFINITY;
            continue;
        }
        int64_t blk = J->block_table[b * J->max_blocks + p / bs];
        int64_t slot = p % bs;
        int64_t base = ((blk * bs + slot) * Hkv + g) * d;
        double s = 0.0;
        for (int c = 0; c < d; ++c)
            s += (double)qrow[c] * kv_elem(J->k_cache, J->kv_dtype, J->k_scale, blk, base + c);
        s *= J->sm_scale;
        score[p] = s;
        if (s > smax)
            smax = s;
    }
    double denom = 0.0;
    for (int64_t p = 0; p < n_vis; ++p) {
        score[p] = exp(score[p] - smax);
        denom += score[p];
    }
    for (int64_t p = 0; p < n_vis; ++p) {
        if (J->tree_mask && p >= L - T && !((anc >> (p - (L - T))) & 1u))
            continue; /* a tree node outside A(t) */
        int64_t blk = J->block_table[b * J->max_blocks + p / bs];
        int64_t slot = p % bs;
        int64_t base = ((blk * bs + slot) * Hkv + g) * d;
        double w = score[p] / denom;
        for (int c = 0; c < d; ++c)
            o[c] += w * kv_elem(J->v_cache, J->kv_dtype, J->v_scale, blk, base + c);
    }
}

typedef struct {
    const attn_job *job;
    int64_t begin, end;
} attn_slice;

static void *attn_worker(void *arg)
{
    const attn_slice *S = (const attn_slice *)arg;
    const attn_job *J = S->job;
    double *score = (double *)malloc(sizeof(double) * ((size_t)J->max_blocks * J->block_size + 1));
    if (!score)
        return (void *)1;
    for (int64_t i = S->begin; i < S->end; ++i) {
        int64_t row = J->rows ? J->rows[i] : i;
        attn_one_row(J, row, score, J->out + i * J->d);
    }
    free(score);
    return NULL;
}

/*
 * Computes the requested output rows into out[nrows][d] (double).
 * rows[i] is the flat row index (b*T + t)*Hq + h; rows == NULL means every row
 * in order (nrows must then be B*T*Hq).  Returns 0, or -1 on bad arguments.
 * Rows with no visible position (L_b < T - t) are NaN.
 */
int oracle_attn_rows_tree(const float *q, const void *k_cache, const void *v_cache,
                          const float *k_scale, const float *v_scale,
                          const int32_t *block_table, const int32_t *context_lens,
                          const uint32_t *tree_mask,
                          int B, int T, int Hq, int Hkv, int d, int block_size,
                          int max_blocks, int kv_dtype, double sm_scale,
                          const int64_t *rows, int64_t nrows, double *out, int nthreads);

int oracle_attn_rows(const float *q, const void *k_cache, const void *v_cache,
                     const float *k_scale, const float *v_scale,
                     const int32_t *block_table, const int32_t *context_lens,
                     int B, int T, int Hq, int Hkv, int d, int block_size,
                     int max_blocks, int kv_dtype, double sm_scale,
                     const int64_t *rows, int64_t nrows, double *out, int nthreads)
{
    return oracle_attn_rows_tree(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, NULL, B, T,
                                 Hq, Hkv, d, block_size, max_blocks, kv_dtype, sm_scale, rows, nrows, out,
                                 nthreads);
}

/*
 * Tree verification ([KV] 8.2 and Q14): the T = N tree nodes are flattened
 * in BFS order into the last N cache positions; node t may attend to the
 * prefix (positions 0 .. L_b - N - 1) and to the nodes of its ancestor set
 * A(t), itself included: bit j of tree_mask[b][t] set iff node j is in A(t).
 * Every set must hold t and no node after t (ancestors precede in BFS order),
 * else -1.  tree_mask == NULL is the chain, A(t) = {0 .. t}.
 */
int oracle_attn_rows_tree(const float *q, const void *k_cache, const void *v_cache,
                          const float *k_scale, const float *v_scale,
                          const int32_t *block_table, const int32_t *context_lens,
                          const uint32_t *tree_mask,
                          int B, int T, int Hq, int Hkv, int d, int block_size,
                          int max_blocks, int kv_dtype, double sm_scale,
                          const int64_t *rows, int64_t nrows, double *out, int nthreads)
{
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out)
        return -1;
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || d < 1 || block_size < 1 || max_blocks < 1)
        return -1;
    if (kv_dtype == OR_KV_FP8_E4M3 && (!k_scale || !v_scale))
        return -1;
    for (int b = 0; b < B; ++b)
        if (context_lens[b] < 0 || context_lens[b] > (int64_t)max_blocks * block_size)
            return -1;
    if (tree_mask) {
        if (T > 32)
            return -1;
        for (int b = 0; b < B; ++b)
            for (int t = 0; t < T; ++t) {
                uint32_t m = tree_mask[b * T + t];
                if (!((m >> t) & 1u) || (t < 31 && (m >> (t + 1))))
                    return -1;
            }
    }
    attn_job J = {q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens,
                  B, T, Hq, Hkv, d, block_size, max_blocks, kv_dtype, sm_scale,
                  rows, nrows, out, NULL, tree_mask};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;
    pthread_t th[256];
    attn_slice sl[256];
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &J;
        sl[i].begin = nrows * i / nthreads;
        sl[i].end = nrows * (i + 1) / nthreads;
    }
    if (nthreads == 1)
        return attn_worker(&sl[0]) ? -1 : 0;
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, attn_worker, &sl[i]);
    for (int i = 0; i < nthreads; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -1;
    }
    return rc;
}

/* ------------------------------------------------------------------- sampler */

/* Target distribution of one verify row: softmax of the fp32 logits, computed
 * with the maximum subtracted ([KV] 7.6 step 3 applies softmax to each target
 * row; temperature 1). */
void oracle_softmax_row(const float *logits, int64_t V, double *p)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j)
        if ((double)logits[j] > m)
            m = (double)logits[j];
    double z = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        p[j] = exp((double)logits[j] - m);
        z += p[j];
    }
    for (int64_t j = 0; j < V; ++j)
        p[j] /= z;
}

/* Target distribution of one verify row at temperature tau ([KV] 7.5 and the
 * answer on temperature there: the sampler-transformed p~ replaces p in the
 * acceptance test, the residual and the bonus draw; p~ is proportional to
 * p^(1/tau), i.e. softmax(logits / tau), computed as exp((l - max) / tau)
 * normalised).  tau = 1 is oracle_softmax_row itself; tau <= 0 reads as the
 * greedy limit: all mass on the first maximal logit. */
void oracle_target_row(const float *logits, int64_t V, double tau, double *p)
{
    if (tau == 1.0) {
        oracle_softmax_row(logits, V, p);
        return;
    }
    double m = -INFINITY;
    int64_t arg = 0;
    for (int64_t j = 0; j < V; ++j)
        if ((double)logits[j] > m) {
            m = (double)logits[j];
            arg = j;
        }
    if (!(tau > 0.0)) {
        for (int64_t j = 0; j < V; ++j)
            p[j] = j == arg ? 1.0 : 0.0;
        return;
    }
    double z = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        p[j] = exp(((double)logits[j] - m) / tau);
        z += p[j];
    }
    for (int64_t j = 0; j < V; ++j)
        p[j] /= z;
}

/* Entry of the ranking used by the top-p truncation: a token and its logit. */
typedef struct {
    float l;
    int64_t j;
} ranked;

static int rank_desc(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->l != y->l)
        return x->l > y->l ? -1 : 1;
    return x->j < y->j ? -1 : (x->j > y->j ? 1 : 0);
}

/* Top-p truncation of a target row ([KV] 7.5 and its answer on top-p: p~ is p
 * cut to p's own top-p set and renormalised; the rejection rule stays exact
 * because p~ is again a distribution).  The set: tokens ranked by their
 * logit (which orders p, as p grows with the logit), a token is kept iff the
 * mass of the tokens ranked strictly above it is below top_p; the tokens of
 * the highest logit are always kept, so top_p <= 0 leaves that group only.
 * Equal logits share one decision.  top_p >= 1 or NaN keeps everything.
 * p (the untruncated row, summing to 1) is truncated and renormalised in
 * place.  Returns 1 if the set is decided within near_eps of top_p (the last
 * kept or the first dropped group), 0 if not, -1 if out of memory. */
int oracle_top_p(const float *logits, int64_t V, double top_p, double near_eps, double *p)
{
    if (!(top_p < 1.0))
        return 0;
    ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)V);
    if (!r)
        return -1;
    for (int64_t j = 0; j < V; ++j) {
        r[j].l = logits[j];
        r[j].j = j;
    }
    qsort(r, (size_t)V, sizeof(ranked), rank_desc);
    double above = 0.0, kept = 0.0;
    int amb = 0;
    int64_t g = 0;
    int first = 1;
    while (g < V) {
        int64_t e = g;
        double mass = 0.0;
        while (e < V && r[e].l == r[g].l)
            mass += p[r[e++].j];
        const int keep = first || above < top_p;
        if (!first && fabs(above - top_p) < near_eps)
            amb = 1;
        if (!keep)
            break;
        kept += mass;
        above += mass;
        first = 0;
        g = e;
    }
    for (int64_t k = g; k < V; ++k)
        p[r[k].j] = 0.0;
    for (int64_t j = 0; j < V; ++j)
        p[j] /= kept;
    free(r);
    return amb;
}

typedef struct {
    const float *target_logits, *draft_probs, *uniforms;
    const int32_t *draft_tokens;
    const float *temperature, *top_p;
    int B, K;
    int64_t V;
    double near_eps;
    int32_t *num_accepted, *out_tokens, *near_pos;
    double *accept_ratio, *resid_mass;
} sample_job;

/*
 * One sequence of the verify sampler ([SD] 3.1; [KV] 7.1-7.3 and 7.6).
 *   Row i of the target logits gives p_i; row i < K verifies draft x_i, row K
 *   is the bonus row.  Draft x_i is accepted with probability
 *   min(1, p_i(x_i)/q_i(x_i)): with the caller's uniform u_i that is the test
 *   u_i * q_i(x_i) < p_i(x_i) (strict, as "rand < r" in [KV] 7.6).
 *   At the first rejection n the replacement is drawn from
 *   max(0, p_n - q_n) / sum(max(0, p_n - q_n)); if all K are accepted the
 *   bonus is drawn from p_K.  Drawing uses u_K and the inverse CDF in
 *   ascending token order: the smallest j whose cumulative weight exceeds
 *   u_K * S.  Should rounding leave no such j, the largest j of positive
 *   weight is taken; should the residual mass S be 0 (only reachable by
 *   rounding, since p <= q everywhere forces p = q), p_n is drawn instead.
 *   Output: n accepted drafts, then the drawn token, then -1 padding.
 *   near_pos = first position whose decision lies within near_eps of its
 *   threshold (acceptance: |u_i - min(1, p/q)|; final draw: u_K within
 *   near_eps of either edge of the chosen token's CDF interval), else -1.
 */
/* p~ of row i of sequence b: temperature, then the top-p cut (skipped for
 * greedy rows, already one-hot).  Returns 1 if the cut is ambiguous. */
static int row_dist(const sample_job *J, int b, int i, double *p)
{
    const double tau = J->temperature ? (double)J->temperature[b] : 1.0;
    const float *lrow = J->target_logits + ((int64_t)b * (J->K + 1) + i) * J->V;
    oracle_target_row(lrow, J->V, tau, p);
    if (!J->top_p || !(tau > 0.0))
        return 0;
    return oracle_top_p(lrow, J->V, (double)J->top_p[b], J->near_eps, p);
}

static void sample_one(const sample_job *J, int b, double *p, double *w)
{
    const int K = J->K;
    const int64_t V = J->V;
    const float *u = J->uniforms + (int64_t)b * (K + 1);
    int n = K;
    int near = -1;

    for (int i = 0; i < K; ++i) {
        const float *qrow = J->draft_probs + ((int64_t)b * K + i) * V;
        if (row_dist(J, b, i, p) && near < 0)
            near = i;
        int x = J->draft_tokens[(int64_t)b * K + i];
        double a = p[x];
        double c = (double)qrow[x];
        double r = c > 0.0 ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
        J->accept_ratio[(int64_t)b * K + i] = r;
        if (near < 0 && fabs((double)u[i] - r) < J->near_eps)
            near = i;
        if (!((double)u[i] * c < a)) {
            n = i;
            break;
        }
    }
    for (int i = n + 1; i < K; ++i)
        J->accept_ratio[(int64_t)b * K + i] = NAN;

    if (row_dist(J, b, n, p) && near < 0)
        near = n;
    double S = 0.0;
    if (n < K) {
        const float *qrow = J->draft_probs + ((int64_t)b * K + n) * V;
        for (int64_t j = 0; j < V; ++j) {
            double r = p[j] - (double)qrow[j];
            w[j] = r > 0.0 ? r : 0.0;
            S += w[j];
        }
    } else {
        for (int64_t j = 0; j < V; ++j) {
            w[j] = p[j];
            S += w[j];
        }
    }
    J->resid_mass[b] = S;
    if (S == 0.0) {
        S = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            w[j] = p[j];
            S += w[j];
        }
    }

    double target = (double)u[K] * S;
    double C = 0.0, Cprev = 0.0;
    int64_t tok = -1;
    for (int64_t j = 0; j < V; ++j) {
        Cprev = C;
        C += w[j];
        if (C > target) {
            tok = j;
            break;
        }
    }
    if (tok < 0) {
        for (int64_t j = V - 1; j >= 0; --j)
            if (w[j] > 0.0) {
                tok = j;
                break;
            }
        Cprev = S;
        C = S;
    }
    if (near < 0 && (fabs((double)u[K] - Cprev / S) < J->near_eps ||
                     fabs((double)u[K] - C / S) < J->near_eps))
        near = n;

    int32_t *ot = J->out_tokens + (int64_t)b * (K + 1);
    for (int i = 0; i < n; ++i)
        ot[i] = J->draft_tokens[(int64_t)b * K + i];
    ot[n] = (int32_t)tok;
    for (int i = n + 1; i <= K; ++i)
        ot[i] = -1;
    J->num_accepted[b] = n;
    J->near_pos[b] = near;
}

typedef struct {
    const sample_job *job;
    int begin, end;
} sample_slice;

static void *sample_worker(void *arg)
{
    const sample_slice *S = (const sample_slice *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)S->job->V);
    double *w = (double *)malloc(sizeof(double) * (size_t)S->job->V);
    if (!p || !w) {
        free(p);
        free(w);
        return (void *)1;
    }
    for (int b = S->begin; b < S->end; ++b)
        sample_one(S->job, b, p, w);
    free(p);
    free(w);
    return NULL;
}

/*
 * The whole sampler for B sequences.  Shapes: target_logits [B][K+1][V],
 * draft_probs [B][K][V], draft_tokens [B][K] (in [0, V)), uniforms [B][K+1];
 * outputs num_accepted [B], out_tokens [B][K+1], accept_ratio [B][K]
 * (positions after the first rejection are NaN), near_pos [B],
 * resid_mass [B] (S before any fallback).  Returns 0, or -1 on bad arguments.
 */
int oracle_sample_t(const float *target_logits, const float *draft_probs,
                    const int32_t *draft_tokens, const float *uniforms, const float *temperature,
                    int B, int K, int64_t V, double near_eps,
                    int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                    int32_t *near_pos, double *resid_mass, int nthreads);

int oracle_sample(const float *target_logits, const float *draft_probs,
                  const int32_t *draft_tokens, const float *uniforms,
                  int B, int K, int64_t V, double near_eps,
                  int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                  int32_t *near_pos, double *resid_mass, int nthreads)
{
    return oracle_sample_t(target_logits, draft_probs, draft_tokens, uniforms, NULL, B, K, V, near_eps,
                           num_accepted, out_tokens, accept_ratio, near_pos, resid_mass, nthreads);
}

int oracle_sample_tp(const float *target_logits, const float *draft_probs,
                     const int32_t *draft_tokens, const float *uniforms, const float *temperature,
                     const float *top_p, int B, int K, int64_t V, double near_eps,
                     int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                     int32_t *near_pos, double *resid_mass, int nthreads);

/* As oracle_sample, with per-sequence temperatures temperature[B] (NULL: 1). */
int oracle_sample_t(const float *target_logits, const float *draft_probs,
                    const int32_t *draft_tokens, const float *uniforms, const float *temperature,
                    int B, int K, int64_t V, double near_eps,
                    int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                    int32_t *near_pos, double *resid_mass, int nthreads)
{
    return oracle_sample_tp(target_logits, draft_probs, draft_tokens, uniforms, temperature, NULL, B, K, V,
                            near_eps, num_accepted, out_tokens, accept_ratio, near_pos, resid_mass, nthreads);
}

/* As oracle_sample_t, with per-sequence top-p values top_p[B] (NULL: none);
 * a top-p decision within near_eps also sets near_pos. */
int oracle_sample_tp(const float *target_logits, const float *draft_probs,
                     const int32_t *draft_tokens, const float *uniforms, const float *temperature,
                     const float *top_p, int B, int K, int64_t V, double near_eps,
                     int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                     int32_t *near_pos, double *resid_mass, int nthreads)
{
    if (!target_logits || !draft_probs || !draft_tokens || !uniforms || !num_accepted ||
        !out_tokens || !accept_ratio || !near_pos || !resid_mass)
        return -1;
    if (B < 1 || K < 1 || V < 1)
        return -1;
    for (int64_t i = 0; i < (int64_t)B * K; ++i)
        if (draft_tokens[i] < 0 || draft_tokens[i] >= V)
            return -1;
    sample_job J = {target_logits, draft_probs, uniforms, draft_tokens, temperature, top_p, B, K, V, near_eps,
                    num_accepted, out_tokens, near_pos, accept_ratio, resid_mass};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > B)
        nthreads = B;
    pthread_t th[256];
    sample_slice sl[256];
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &J;
        sl[i].begin = (int)((int64_t)B * i / nthreads);
        sl[i].end = (int)((int64_t)B * (i + 1) / nthreads);
    }
    if (nthreads == 1)
        return sample_worker(&sl[0]) ? -1 : 0;
    int rc = 0;
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, sample_worker, &sl[i]);
    for (int i = 0; i < nthreads; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -1;
    }
    return rc;
}

/* ------------------------------------------------------- typical acceptance
 *
 * Typical acceptance ([SD] 9.1; [KV] 8.2 and Q18): not exact.  Draft x_i is
 * accepted iff the target's own probability of it exceeds an entropy-based
 * threshold, p~_i(x_i) > min(eps, delta * exp(-H(p~_i))), H the entropy of
 * the (tempered) target row in nats; the draft probabilities take no part.
 * Reading where the pages stop: the comparison is strict ("exceeds"); at the
 * first rejection n (or n = K) the next token is drawn from the target row
 * p~_n itself with the last uniform, by the chain's inverse CDF -- the
 * target's own prediction at that position, with no residual since nothing
 * is conditioned on the draft.
 */

/* Entropy -sum p log p of a distribution, in nats (terms with p = 0 add 0). */
double oracle_entropy(const double *p, int64_t V)
{
    double h = 0.0;
    for (int64_t j = 0; j < V; ++j)
        if (p[j] > 0.0)
            h -= p[j] * log(p[j]);
    return h;
}

typedef struct {
    const float *target_logits, *uniforms, *temperature;
    const int32_t *draft_tokens;
    double eps, delta;
    int B, K;
    int64_t V;
    double near_eps;
    int32_t *num_accepted, *out_tokens, *near_pos;
    double *p_draft, *threshold;
} typical_job;

static void typical_one(const typical_job *J, int b, double *p)
{
    const int K = J->K;
    const int64_t V = J->V;
    const float *u = J->uniforms + (int64_t)b * (K + 1);
    const double tau = J->temperature ? (double)J->temperature[b] : 1.0;
    int n = K, near = -1;
    for (int i = 0; i < K; ++i) {
        oracle_target_row(J->target_logits + ((int64_t)b * (K + 1) + i) * V, V, tau, p);
        const double th = fmin(J->eps, J->delta * exp(-oracle_entropy(p, V)));
        const int x = J->draft_tokens[(int64_t)b * K + i];
        J->p_draft[(int64_t)b * K + i] = p[x];
        J->threshold[(int64_t)b * K + i] = th;
        if (near < 0 && fabs(p[x] - th) < J->near_eps)
            near = i;
        if (!(p[x] > th)) {
            n = i;
            break;
        }
    }
    for (int i = n + 1; i < K; ++i) {
        J->p_draft[(int64_t)b * K + i] = NAN;
        J->threshold[(int64_t)b * K + i] = NAN;
    }
    oracle_target_row(J->target_logits + ((int64_t)b * (K + 1) + n) * V, V, tau, p);
    double S = 0.0;
    for (int64_t j = 0; j < V; ++j)
        S += p[j];
    const double target = (double)u[K] * S;
    double cum = 0.0, cum_prev = 0.0;
    int64_t tok = -1;
    for (int64_t j = 0; j < V; ++j) {
        cum_prev = cum;
        cum += p[j];
        if (cum > target) {
            tok = j;
            break;
        }
    }
    if (tok < 0) {
        for (int64_t j = V - 1; j >= 0; --j)
            if (p[j] > 0.0) {
                tok = j;
                break;
            }
        cum_prev = S;
        cum = S;
    }
    if (near < 0 && (fabs((double)u[K] - cum_prev / S) < J->near_eps || fabs((double)u[K] - cum / S) < J->near_eps))
        near = n;
    int32_t *ot = J->out_tokens + (int64_t)b * (K + 1);
    for (int i = 0; i < n; ++i)
        ot[i] = J->draft_tokens[(int64_t)b * K + i];
    ot[n] = (int32_t)tok;
    for (int i = n + 1; i <= K; ++i)
        ot[i] = -1;
    J->num_accepted[b] = n;
    J->near_pos[b] = near;
}

typedef struct {
    const typical_job *job;
    int begin, end;
} typical_slice;

static void *typical_worker(void *arg)
{
    const typical_slice *S = (const typical_slice *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)S->job->V);
    if (!p)
        return (void *)1;
    for (int b = S->begin; b < S->end; ++b)
        typical_one(S->job, b, p);
    free(p);
    return NULL;
}

/*
 * Typical acceptance for B sequences.  Shapes as oracle_sample (no draft
 * probabilities); temperature [B] or NULL.  Outputs: num_accepted [B],
 * out_tokens [B][K+1], p_draft [B][K] (p~_i(x_i)) and threshold [B][K]
 * (min(eps, delta exp(-H))) for every tested position, NaN after the first
 * rejection; near_pos [B]: first position whose test lies within near_eps of
 * its threshold, or whose draw lies within near_eps of a CDF edge.
 */
int oracle_sample_typical(const float *target_logits, const int32_t *draft_tokens, const float *uniforms,
                          const float *temperature, double eps, double delta, int B, int K, int64_t V,
                          double near_eps, int32_t *num_accepted, int32_t *out_tokens, double *p_draft,
                          double *threshold, int32_t *near_pos, int nthreads)
{
    if (!target_logits || !draft_tokens || !uniforms || !num_accepted || !out_tokens || !p_draft || !threshold ||
        !near_pos)
        return -1;
    if (B < 1 || K < 1 || V < 1)
        return -1;
    for (int64_t i = 0; i < (int64_t)B * K; ++i)
        if (draft_tokens[i] < 0 || draft_tokens[i] >= V)
            return -1;
    typical_job J = {target_logits, uniforms, temperature, draft_tokens, eps, delta, B, K, V, near_eps,
                     num_accepted, out_tokens, near_pos, p_draft, threshold};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > B)
        nthreads = B;
    pthread_t th[256];
    typical_slice sl[256];
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &J;
        sl[i].begin = (int)((int64_t)B * i / nthreads);
        sl[i].end = (int)((int64_t)B * (i + 1) / nthreads);
    }
    if (nthreads == 1)
        return typical_worker(&sl[0]) ? -1 : 0;
    int rc = 0;
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, typical_worker, &sl[i]);
    for (int i = 0; i < nthreads; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -1;
    }
    return rc;
}

/* ------------------------------------------------------------ tree sampler
 *
 * Verification of a draft tree ([KV] 8.2 and Q14: the tree's nodes are
 * flattened in BFS order and scored by one target forward; exact
 * verification keeps the rejection rule of [SD] 3.1 and [KV] 7.1-7.3).
 *
 * Inputs per sequence: N nodes in BFS order, parents[0] < 0 (the root is the
 * last committed token), 0 <= parents[c] < c otherwise; tokens[c] the token
 * of node c (tokens[0] unused); target row c = logits after node c's path;
 * draft row c = the distribution q_c the children of c were drawn from;
 * uniforms[c] (c >= 1) tests node c, uniforms[0] drives the final draw.
 *
 * Reading for siblings (the pages name exact tree verification but give no
 * rule for several candidates at one node): the children of the current
 * node are tried in BFS order, each against the target as left by the
 * siblings rejected before it, the residual step of [SD] 3.1 applied once
 * per rejection: p_1 = p, p_{k+1} = norm(max(0, p_k - q)).  Unnormalised,
 * p_k = max(0, p - C_{k-1} q) / Z_k with C_0 = 0, Z_1 = 1,
 * Z_k = sum_j max(0, p_j - C_{k-1} q_j) and C_k = C_{k-1} + Z_k.  Child k with
 * token x is accepted iff u * q(x) < p_k(x); the walk then moves to it.  When
 * no child is accepted (or there is none) the final token is drawn from the
 * current residual max(0, p - C q) (p itself at a leaf or with no
 * rejection), by the same inverse CDF and fallbacks as the chain.  A chain
 * tree is exactly the chain sampler.
 */
typedef struct {
    const float *target_logits, *draft_probs, *uniforms;
    const int32_t *tokens, *parents;
    int B, N;
    int64_t V;
    double near_eps;
    int32_t *num_accepted, *out_tokens, *path, *near_pos;
    double *accept_ratio;
} tree_job;

static void tree_one(const tree_job *J, int b, double *p, double *w)
{
    const int N = J->N;
    const int64_t V = J->V;
    const int32_t *par = J->parents + (int64_t)b * N;
    const int32_t *tok = J->tokens + (int64_t)b * N;
    const float *u = J->uniforms + (int64_t)b * N;
    int32_t *ot = J->out_tokens + (int64_t)b * N;
    int32_t *pth = J->path + (int64_t)b * N;
    double *ar = J->accept_ratio + (int64_t)b * N;
    for (int i = 0; i < N; ++i) {
        ot[i] = -1;
        pth[i] = -1;
        ar[i] = NAN;
    }
    int node = 0, depth = 0, near = -1;
    double C = 0.0;
    const float *qrow = NULL;
    for (;;) {
        oracle_softmax_row(J->target_logits + ((int64_t)b * N + node) * V, V, p);
        qrow = J->draft_probs + ((int64_t)b * N + node) * V;
        C = 0.0;
        int next = -1;
        for (int c = node + 1; c < N; ++c) {
            if (par[c] != node)
                continue;
            const int x = tok[c];
            const double qx = (double)qrow[x];
            double a;
            double Z = 1.0;
            if (C == 0.0) {
                a = p[x];
            } else {
                Z = 0.0;
                for (int64_t j = 0; j < V; ++j) {
                    double r = p[j] - C * (double)qrow[j];
                    Z += r > 0.0 ? r : 0.0;
                }
                double rx = p[x] - C * qx;
                a = (Z > 0.0 && rx > 0.0) ? rx / Z : 0.0;
            }
            const double ratio = qx > 0.0 ? fmin(1.0, a / qx) : (a > 0.0 ? 1.0 : 0.0);
            ar[c] = ratio;
            if (near < 0 && fabs((double)u[c] - ratio) < J->near_eps)
                near = depth;
            if ((double)u[c] * qx < a) {
                next = c;
                break;
            }
            C += Z;
        }
        if (next < 0)
            break;
        pth[depth] = next;
        ot[depth] = tok[next];
        ++depth;
        node = next;
    }

    double S = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double r = C == 0.0 ? p[j] : p[j] - C * (double)qrow[j];
        w[j] = r > 0.0 ? r : 0.0;
        S += w[j];
    }
    if (S == 0.0) {
        for (int64_t j = 0; j < V; ++j) {
            w[j] = p[j];
            S += w[j];
        }
    }
    double target = (double)u[0] * S;
    double Cum = 0.0, Cprev = 0.0;
    int64_t pick = -1;
    for (int64_t j = 0; j < V; ++j) {
        Cprev = Cum;
        Cum += w[j];
        if (Cum > target) {
            pick = j;
            break;
        }
    }
    if (pick < 0) {
        for (int64_t j = V - 1; j >= 0; --j)
            if (w[j] > 0.0) {
                pick = j;
                break;
            }
        Cprev = S;
        Cum = S;
    }
    if (near < 0 && (fabs((double)u[0] - Cprev / S) < J->near_eps || fabs((double)u[0] - Cum / S) < J->near_eps))
        near = depth;
    ot[depth] = (int32_t)pick;
    J->num_accepted[b] = depth;
    J->near_pos[b] = near;
}

typedef struct {
    const tree_job *job;
    int begin, end;
} tree_slice;

static void *tree_worker(void *arg)
{
    const tree_slice *S = (const tree_slice *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)S->job->V);
    double *w = (double *)malloc(sizeof(double) * (size_t)S->job->V);
    if (!p || !w) {
        free(p);
        free(w);
        return (void *)1;
    }
    for (int b = S->begin; b < S->end; ++b)
        tree_one(S->job, b, p, w);
    free(p);
    free(w);
    return NULL;
}

/*
 * The tree sampler for B sequences of N nodes each.  Shapes: target_logits
 * and draft_probs [B][N][V], tokens, parents, uniforms [B][N].  Outputs:
 * num_accepted [B] (accepted nodes, the root not counted), out_tokens [B][N]
 * (the accepted nodes' tokens, then the drawn token, then -1), path [B][N]
 * (the accepted node ids in order, then -1), accept_ratio [B][N] (the
 * min(1, p_k/q) of every tested node, NaN elsewhere), near_pos [B] (first
 * output position decided within near_eps, else -1).  Returns 0, or -1 on
 * bad arguments (a parent that does not precede its child, a token out of
 * range).
 */
int oracle_sample_tree(const float *target_logits, const float *draft_probs, const int32_t *tokens,
                       const int32_t *parents, const float *uniforms, int B, int N, int64_t V, double near_eps,
                       int32_t *num_accepted, int32_t *out_tokens, int32_t *path, double *accept_ratio,
                       int32_t *near_pos, int nthreads)
{
    if (!target_logits || !draft_probs || !tokens || !parents || !uniforms || !num_accepted || !out_tokens ||
        !path || !accept_ratio || !near_pos)
        return -1;
    if (B < 1 || N < 1 || V < 1)
        return -1;
    for (int b = 0; b < B; ++b) {
        if (parents[(int64_t)b * N] >= 0)
            return -1;
        for (int c = 1; c < N; ++c) {
            int32_t pc = parents[(int64_t)b * N + c], x = tokens[(int64_t)b * N + c];
            if (pc < 0 || pc >= c || x < 0 || x >= V)
                return -1;
        }
    }
    tree_job J = {target_logits, draft_probs, uniforms, tokens, parents, B, N, V, near_eps,
                  num_accepted, out_tokens, path, near_pos, accept_ratio};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > B)
        nthreads = B;
    pthread_t th[256];
    tree_slice sl[256];
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &J;
        sl[i].begin = (int)((int64_t)B * i / nthreads);
        sl[i].end = (int)((int64_t)B * (i + 1) / nthreads);
    }
    if (nthreads == 1)
        return tree_worker(&sl[0]) ? -1 : 0;
    int rc = 0;
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, tree_worker, &sl[i]);
    for (int i = 0; i < nthreads; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -1;
    }
    return rc;
}

/* Ancestor sets of a BFS-ordered tree ([KV] 8.2, Q14): bit j of masks[c] is
 * set iff node j lies on the path from the root to c, c included.  Returns
 * 0, or -1 if a parent does not precede its child or N > 32. */
int oracle_tree_masks(const int32_t *parents, int B, int N, uint32_t *masks)
{
    if (N < 1 || N > 32)
        return -1;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * N;
        uint32_t *m = masks + (int64_t)b * N;
        if (par[0] >= 0)
            return -1;
        m[0] = 1u;
        for (int c = 1; c < N; ++c) {
            if (par[c] < 0 || par[c] >= c)
                return -1;
            m[c] = m[par[c]] | (1u << c);
        }
    }
    return 0;
}

/* ------------------------------------------------------- paged append / rollback
 *
 * Appending the verify positions to the paged cache and truncating it after
 * the sampler ([KV] 6.1 naive append, 6.2 paged data structure, 7.6 the loop
 * and its note that a paged cache rolls back by changing table entries;
 * [L10] 9.2).
 */

/* float -> bfloat16 bits, round to nearest, ties to even, from the format
 * definition: the 16 dropped fraction bits decide; NaN stays NaN (quiet). */
uint16_t oracle_encode_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16, drop = u & 0xFFFFu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u;
    return (uint16_t)keep;
}

/* float -> OCP E4M3 ("fn") code for the value x / scale.  The quotient is
 * rounded to float first (as a float division does), then mapped to the
 * nearest E4M3 value by direct search over the 127 non-negative finite codes;
 * a tie goes to the code with an even last fraction bit.  Magnitudes above
 * 448 (infinity included) saturate to 448; NaN maps to the NaN code. */
uint8_t oracle_encode_e4m3(float x, float scale)
{
    float qf = x / scale;
    if (isnan(qf))
        return 0x7F;
    uint8_t sign = signbit(qf) ? 0x80 : 0x00;
    double a = fabs((double)qf);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bestd = a;   /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(oracle_decode_e4m3((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* k_new, v_new [B][T][Hkv][d] float; caches [num_blocks][16][Hkv][d] of
 * kv_dtype, written in place.  For every (b, t, g): position
 * p = L_b - T + t, page = block_table[b][p / 16], slot = p % 16.  Returns -1
 * (writing nothing) if any position or page id is out of range. */
int oracle_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache,
                     const float *k_scale, const float *v_scale, const int32_t *block_table,
                     const int32_t *context_lens, int B, int T, int Hkv, int d, int max_blocks,
                     int num_blocks, int kv_dtype)
{
    for (int b = 0; b < B; ++b) {
        if (context_lens[b] < T || context_lens[b] > max_blocks * 16)
            return -1;
        for (int t = 0; t < T; ++t) {
            int p = context_lens[b] - T + t;
            int page = block_table[(int64_t)b * max_blocks + p / 16];
            if (page < 0 || page >= num_blocks)
                return -1;
        }
    }
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            int p = context_lens[b] - T + t;
            int64_t page = block_table[(int64_t)b * max_blocks + p / 16];
            int slot = p % 16;
            for (int g = 0; g < Hkv; ++g)
                for (int c = 0; c < d; ++c) {
                    int64_t src = (((int64_t)b * T + t) * Hkv + g) * d + c;
                    int64_t dst = ((page * 16 + slot) * Hkv + g) * d + c;
                    for (int which = 0; which < 2; ++which) {
                        const float x = which ? v_new[src] : k_new[src];
                        void *cache = which ? v_cache : k_cache;
                        if (kv_dtype == OR_KV_F32)
                            ((float *)cache)[dst] = x;
                        else if (kv_dtype == OR_KV_BF16)
                            ((uint16_t *)cache)[dst] = oracle_encode_bf16(x);
                        else
                            ((uint8_t *)cache)[dst] =
                                oracle_encode_e4m3(x, which ? v_scale[page] : k_scale[page]);
                    }
                }
        }
    return 0;
}

/* After the sampler: keep the last committed token and the n_b accepted
 * drafts of the T = K + 1 verify positions, i.e. L_b <- L_b - K + n_b, and
 * report the pages the shorter context still uses, ceil(L_b / 16). */
void oracle_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K)
{
    for (int b = 0; b < B; ++b) {
        int L = context_lens[b] - K + num_accepted[b];
        context_lens[b] = L;
        pages_in_use[b] = (L + 15) / 16;
    }
}

/* ------------------------------------------------------------- tree commit
 *
 * After tree verification ([KV] 8.2; the note of [KV] 7.6 that a paged cache
 * rolls back by editing its bookkeeping): the sequence keeps the root (the
 * last committed token) and the n accepted nodes of the path, in path order,
 * at consecutive positions.  With L the length including the N nodes and
 * base = L - N (the root's position), accepted node path[i] moves from
 * position base + path[i] to base + 1 + i (all sources are read before any
 * destination is written), and L becomes base + 1 + n; pages_in_use =
 * ceil(L / 16).  Values are copied; for E4M3 storage a value that changes
 * page is re-encoded for the destination page: decode(code) * scale_src
 * rounded to float, then encoded as the append encodes (x / scale_dst in
 * float, nearest even, saturating).  A chain path (path[i] = i + 1) moves
 * nothing and is the chain's rollback with K = N - 1.
 */
int oracle_tree_commit(const int32_t *path, const int32_t *num_accepted, void *k_cache, void *v_cache,
                       const float *k_scale, const float *v_scale, const int32_t *block_table,
                       int32_t *context_lens, int32_t *pages_in_use, int B, int N, int Hkv, int d,
                       int max_blocks, int num_blocks, int kv_dtype)
{
    const size_t esz = kv_dtype == OR_KV_F32 ? 4 : (kv_dtype == OR_KV_BF16 ? 2 : 1);
    for (int b = 0; b < B; ++b) {
        const int L = context_lens[b], n = num_accepted[b];
        if (L < N || L > max_blocks * 16 || n < 0 || n > N - 1)
            return -1;
        for (int i = 0; i < n; ++i) {
            const int c = path[(int64_t)b * N + i];
            if (c < 1 || c > N - 1 || (i > 0 && c <= path[(int64_t)b * N + i - 1]))
                return -1;
        }
        for (int p = L - N; p < L; ++p) {
            const int page = block_table[(int64_t)b * max_blocks + p / 16];
            if (page < 0 || page >= num_blocks)
                return -1;
        }
    }
    const size_t row = (size_t)Hkv * d;
    unsigned char *tmp = (unsigned char *)malloc(2 * (size_t)N * row * esz + 1);
    if (!tmp)
        return -1;
    for (int b = 0; b < B; ++b) {
        const int L = context_lens[b], n = num_accepted[b], base = L - N;
        /* read every source row first */
        for (int i = 0; i < n; ++i) {
            const int p = base + path[(int64_t)b * N + i];
            const int64_t page = block_table[(int64_t)b * max_blocks + p / 16];
            const size_t off = ((size_t)page * 16 + p % 16) * row * esz;
            memcpy(tmp + (2 * (size_t)i) * row * esz, (unsigned char *)k_cache + off, row * esz);
            memcpy(tmp + (2 * (size_t)i + 1) * row * esz, (unsigned char *)v_cache + off, row * esz);
        }
        for (int i = 0; i < n; ++i) {
            const int ps = base + path[(int64_t)b * N + i], pd = base + 1 + i;
            const int64_t pgs = block_table[(int64_t)b * max_blocks + ps / 16];
            const int64_t pgd = block_table[(int64_t)b * max_blocks + pd / 16];
            const size_t off = ((size_t)pgd * 16 + pd % 16) * row * esz;
            for (int which = 0; which < 2; ++which) {
                const unsigned char *src = tmp + (2 * (size_t)i + which) * row * esz;
                unsigned char *dst = (unsigned char *)(which ? v_cache : k_cache) + off;
                if (kv_dtype != OR_KV_FP8_E4M3 || pgs == pgd) {
                    memcpy(dst, src, row * esz);
                } else {
                    const float ss = which ? v_scale[pgs] : k_scale[pgs];
                    const float sd = which ? v_scale[pgd] : k_scale[pgd];
                    for (size_t e = 0; e < row; ++e) {
                        const float x = (float)oracle_decode_e4m3(src[e]) * ss;
                        dst[e] = oracle_encode_e4m3(x, sd);
                    }
                }
            }
        }
        context_lens[b] = base + 1 + n;
        if (pages_in_use)
            pages_in_use[b] = (base + 1 + n + 15) / 16;
    }
    free(tmp);
    return 0;
}

