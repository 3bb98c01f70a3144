/*
 * Host-sanitizer driver for the CPU oracle (test infrastructure).  Built
 * together with oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py, it calls every
 * entry point of the oracle on small seeded inputs (several threads where the
 * oracle splits work) and checks the return codes.  Any out-of-bounds access,
 * leak or undefined operation aborts the run with the sanitizer's report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_decode_bf16(uint16_t bits);
double oracle_decode_e4m3(uint8_t bits);
uint16_t oracle_encode_bf16(float x);
uint8_t oracle_encode_e4m3(float x, float scale);
int oracle_attn_rows(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                     const float *v_scale, const int32_t *block_table, const int32_t *context_lens, int B, int T,
                     int Hq, int Hkv, int d, int block_size, int max_blocks, int kv_dtype, double sm_scale,
                     const int64_t *rows, int64_t nrows, double *out, int nthreads);
int oracle_attn_rows_tree(const float *q, const void *k_cache, const void *v_cache, const float *k_scale,
                          const float *v_scale, const int32_t *block_table, const int32_t *context_lens,
                          const uint32_t *tree_mask, int B, int T, int Hq, int Hkv, int d, int block_size,
                          int max_blocks, int kv_dtype, double sm_scale, const int64_t *rows, int64_t nrows,
                          double *out, int nthreads);
void oracle_softmax_row(const float *logits, int64_t V, double *p);
void oracle_target_row(const float *logits, int64_t V, double tau, double *p);
int oracle_top_p(const float *logits, int64_t V, double top_p, double near_eps, double *p);
int oracle_sample(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                  const float *uniforms, int B, int K, int64_t V, double near_eps, int32_t *num_accepted,
                  int32_t *out_tokens, double *accept_ratio, int32_t *near_pos, double *resid_mass, int nthreads);
int oracle_sample_tp(const float *target_logits, const float *draft_probs, const int32_t *draft_tokens,
                     const float *uniforms, const float *temperature, const float *top_p, int B, int K, int64_t V,
                     double near_eps, int32_t *num_accepted, int32_t *out_tokens, double *accept_ratio,
                     int32_t *near_pos, double *resid_mass, int nthreads);
double oracle_entropy(const double *p, int64_t V);
int oracle_sample_typical(const float *target_logits, const int32_t *draft_tokens, const float *uniforms,
                          const float *temperature, double eps, double delta, int B, int K, int64_t V,
                          double near_eps, int32_t *num_accepted, int32_t *out_tokens, double *p_draft,
                          double *threshold, int32_t *near_pos, int nthreads);
int oracle_sample_tree(const float *target_logits, const float *draft_probs, const int32_t *tokens,
                       const int32_t *parents, const float *uniforms, int B, int N, int64_t V, double near_eps,
                       int32_t *num_accepted, int32_t *out_tokens, int32_t *path, double *accept_ratio,
                       int32_t *near_pos, int nthreads);
int oracle_tree_masks(const int32_t *parents, int B, int N, uint32_t *masks);
int oracle_kv_append(const float *k_new, const float *v_new, void *k_cache, void *v_cache, const float *k_scale,
                     const float *v_scale, const int32_t *block_table, const int32_t *context_lens, int B, int T,
                     int Hkv, int d, int max_blocks, int num_blocks, int kv_dtype);
void oracle_rollback(const int32_t *num_accepted, int32_t *context_lens, int32_t *pages_in_use, int B, int K);
int oracle_tree_commit(const int32_t *path, const int32_t *num_accepted, void *k_cache, void *v_cache,
                       const float *k_scale, const float *v_scale, const int32_t *block_table,
                       int32_t *context_lens, int32_t *pages_in_use, int B, int N, int Hkv, int d, int max_blocks,
                       int num_blocks, int kv_dtype);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double urand(void) /* splitmix64 -> [0, 1) */
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static float nrand(void) { return (float)(sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307179586 * urand())); }

static int g_fail = 0;
#define CHECK(cond, what)                                                                                    \
    do {                                                                                                     \
        if (!(cond)) {                                                                                       \
            fprintf(stderr, "FAIL: %s\n", what);                                                             \
            g_fail = 1;                                                                                      \
        }                                                                                                    \
    } while (0)

static void run_attention(int kv_dtype, int tree)
{
    const int B = 3, T = tree ? 6 : 4, Hkv = 2, G = 4, Hq = Hkv * G, d = 16, bs = 16;
    const int lens[3] = {T, 37, 100};
    const int max_blocks = 7, num_blocks = 3 * max_blocks + 1;
    const size_t esz = kv_dtype == 0 ? 4 : (kv_dtype == 1 ? 2 : 1);
    const size_t per_block = (size_t)bs * Hkv * d;
    float *q = malloc(sizeof(float) * B * T * Hq * d);
    unsigned char *kc = malloc(esz * per_block * num_blocks), *vc = malloc(esz * per_block * num_blocks);
    float *ks = malloc(sizeof(float) * num_blocks), *vs = malloc(sizeof(float) * num_blocks);
    int32_t *table = malloc(sizeof(int32_t) * B * max_blocks);
    for (int i = 0; i < B * T * Hq * d; ++i)
        q[i] = nrand();
    for (size_t i = 0; i < per_block * num_blocks; ++i) {
        const float a = nrand(), b = nrand();
        if (kv_dtype == 0) {
            ((float *)kc)[i] = a;
            ((float *)vc)[i] = b;
        } else if (kv_dtype == 1) {
            ((uint16_t *)kc)[i] = oracle_encode_bf16(a);
            ((uint16_t *)vc)[i] = oracle_encode_bf16(b);
        } else {
            kc[i] = oracle_encode_e4m3(a, 0.01f);
            vc[i] = oracle_encode_e4m3(b, 0.01f);
        }
    }
    for (int i = 0; i < num_blocks; ++i)
        ks[i] = vs[i] = 0.01f;
    for (int i = 0; i < B * max_blocks; ++i)
        table[i] = i % (num_blocks - 1);
    uint32_t masks[3 * 6];
    if (tree) {
        const int32_t par[6] = {-1, 0, 0, 1, 1, 2};
        int32_t parents[3 * 6];
        for (int b = 0; b < B; ++b)
            memcpy(parents + 6 * b, par, sizeof(par));
        CHECK(oracle_tree_masks(parents, B, 6, masks) == 0, "tree masks");
    }
    const int64_t nrows = (int64_t)B * T * Hq;
    double *out = malloc(sizeof(double) * nrows * d);
    int rc = oracle_attn_rows_tree(q, kc, vc, ks, vs, table, lens, tree ? masks : NULL, B, T, Hq, Hkv, d, bs,
                                   max_blocks, kv_dtype, 0.25, NULL, nrows, out, 4);
    CHECK(rc == 0, "attention rows");
    for (int64_t i = 0; i < nrows * d; ++i)
        CHECK(isfinite(out[i]), "attention output finite");
    int64_t rows[5] = {0, 7, nrows - 1, 13, 40};
    rc = oracle_attn_rows(q, kc, vc, ks, vs, table, lens, B, T, Hq, Hkv, d, bs, max_blocks, kv_dtype, 0.25, rows, 5,
                          out, 2);
    CHECK(rc == 0, "attention selected rows");
    free(q);
    free(kc);
    free(vc);
    free(ks);
    free(vs);
    free(table);
    free(out);
}

static void run_sampler(void)
{
    const int B = 4, K = 3;
    const int64_t V = 777;
    float *logits = malloc(sizeof(float) * B * (K + 1) * V), *probs = malloc(sizeof(float) * B * K * V);
    int32_t tokens[4 * 3];
    float uniforms[4 * 4], temp[4] = {1.0f, 0.7f, 0.0f, 1.3f}, topp[4] = {1.0f, 0.9f, 0.5f, 0.95f};
    for (int64_t i = 0; i < B * (K + 1) * V; ++i)
        logits[i] = 2.0f * nrand();
    for (int r = 0; r < B * K; ++r) {
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v)
            s += (probs[r * V + v] = (float)urand());
        for (int64_t v = 0; v < V; ++v)
            probs[r * V + v] = (float)(probs[r * V + v] / s);
        tokens[r] = (int32_t)(urand() * V);
    }
    for (int i = 0; i < B * (K + 1); ++i)
        uniforms[i] = (float)urand();
    int32_t na[4], out_tok[4 * 4], near[4];
    double ratio[4 * 3], resid[4], pdraft[4 * 3], thr[4 * 3];
    CHECK(oracle_sample(logits, probs, tokens, uniforms, B, K, V, 1e-6, na, out_tok, ratio, near, resid, 3) == 0,
          "sample");
    CHECK(oracle_sample_tp(logits, probs, tokens, uniforms, temp, topp, B, K, V, 1e-6, na, out_tok, ratio, near,
                           resid, 2) == 0,
          "sample with temperature and top-p");
    CHECK(oracle_sample_typical(logits, tokens, uniforms, temp, 0.3, 0.09, B, K, V, 1e-6, na, out_tok, pdraft, thr,
                                near, 2) == 0,
          "typical acceptance");
    double *p = malloc(sizeof(double) * V);
    oracle_softmax_row(logits, V, p);
    CHECK(isfinite(oracle_entropy(p, V)), "entropy");
    oracle_target_row(logits, V, 0.8, p);
    CHECK(oracle_top_p(logits, V, 0.9, 1e-6, p) >= 0, "top-p");
    free(p);
    /* tree: 6 nodes, BFS parents */
    const int N = 6;
    const int32_t par[6] = {-1, 0, 0, 1, 1, 2};
    float *tl = malloc(sizeof(float) * B * N * V), *tp = malloc(sizeof(float) * B * N * V);
    int32_t parents[4 * 6], ttok[4 * 6], path[4 * 6], tout[4 * 6];
    float tu[4 * 6];
    double tratio[4 * 6];
    for (int64_t i = 0; i < B * N * V; ++i)
        tl[i] = 2.0f * nrand();
    for (int r = 0; r < B * N; ++r) {
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v)
            s += (tp[r * V + v] = (float)urand());
        for (int64_t v = 0; v < V; ++v)
            tp[r * V + v] = (float)(tp[r * V + v] / s);
        parents[r] = par[r % N];
        ttok[r] = (int32_t)(urand() * V);
        tu[r] = (float)urand();
    }
    CHECK(oracle_sample_tree(tl, tp, ttok, parents, tu, B, N, V, 1e-6, na, tout, path, tratio, near, 3) == 0,
          "tree sampler");
    free(tl);
    free(tp);
    free(logits);
    free(probs);
}

static void run_cache(int kv_dtype)
{
    const int B = 2, T = 5, Hkv = 2, d = 8, max_blocks = 4, num_blocks = 9;
    const size_t esz = kv_dtype == 0 ? 4 : (kv_dtype == 1 ? 2 : 1);
    const size_t cache = (size_t)num_blocks * 16 * Hkv * d;
    unsigned char *kc = calloc(cache, esz), *vc = calloc(cache, esz);
    float ks[9], vs[9];
    for (int i = 0; i < num_blocks; ++i)
        ks[i] = vs[i] = 0.05f;
    int32_t table[2 * 4] = {0, 1, 2, 3, 4, 5, 6, 7};
    int32_t lens[2] = {21, 50};
    float *kn = malloc(sizeof(float) * B * T * Hkv * d), *vn = malloc(sizeof(float) * B * T * Hkv * d);
    for (int i = 0; i < B * T * Hkv * d; ++i) {
        kn[i] = nrand();
        vn[i] = nrand();
    }
    CHECK(oracle_kv_append(kn, vn, kc, vc, ks, vs, table, lens, B, T, Hkv, d, max_blocks, num_blocks, kv_dtype) == 0,
          "kv append");
    const int32_t path[2 * 5] = {2, 4, -1, -1, -1, 1, -1, -1, -1, -1};
    const int32_t nacc[2] = {2, 1};
    int32_t pages[2];
    CHECK(oracle_tree_commit(path, nacc, kc, vc, ks, vs, table, lens, pages, B, T, Hkv, d, max_blocks, num_blocks,
                             kv_dtype) == 0,
          "tree commit");
    int32_t lens2[2] = {21, 50}, pages2[2];
    oracle_rollback(nacc, lens2, pages2, B, T - 1);
    free(kc);
    free(vc);
    free(kn);
    free(vn);
}

int main(void)
{
    for (uint32_t c = 0; c < 65536; ++c)
        (void)oracle_decode_bf16((uint16_t)c);
    for (uint32_t c = 0; c < 256; ++c)
        (void)oracle_decode_e4m3((uint8_t)c);
    for (int kv = 0; kv < 3; ++kv) {
        run_attention(kv, 0);
        run_attention(kv, 1);
        run_cache(kv);
    }
    run_sampler();
    if (g_fail)
        return 1;
    printf("ok\n");
    return 0;
}
