/*
 * Runs every function of the CPU oracle (oracle/ddtree_oracle.c) on small
 * seeded inputs -- ragged, degenerate and malformed ones included -- so that
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer sees every
 * path: out-of-bounds reads or writes, signed overflow, bad shifts and
 * misaligned loads end the run with a report. The results are also checked
 * for the structural facts every tree and walk must have (the values
 * themselves are pinned by the Python tests).
 *
 * Built and run by tests/test_sanitize_cpu.py:
 *   gcc -std=c11 -O1 -g -fopenmp -ffp-contract=off
 *       -fsanitize=address,undefined -fno-sanitize-recover=all
 *       oracle_driver.c ../../oracle/ddtree_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_row_topk(const void *row, int dtype, int V, int K, float tau, int32_t *topk_tok,
                    float *topk_lp, float *out_m, uint64_t *out_S, float *out_lse);
int oracle_tree(const int32_t *topk_tok, const float *topk_lp, int L, int K, int N,
                int32_t root_token, int32_t *tokens, int32_t *parents, int32_t *depths,
                float *scores);
void oracle_mask(const int32_t *parents, int num_nodes, int T, uint64_t *mask);
void oracle_build(const void *logits, int dtype, const int32_t *root_tokens, int batch, int L,
                  int V, int K, int N, float tau, int32_t *tokens, int32_t *parents,
                  int32_t *depths, float *scores, int32_t *num_nodes, uint64_t *mask,
                  int32_t *topk_tok, float *topk_lp, int32_t *status, float *row_m,
                  uint64_t *row_S, float *row_lse);
void oracle_attn_rows(const void *q, const void *k, const void *v, int dtype,
                      const int64_t *kv_offsets, const int32_t *prefix_lens,
                      const int32_t *num_nodes, const uint64_t *mask, int T, int Hq, int Hkv,
                      int D, int64_t total_rows, double scale, const int32_t *sel, int nsel,
                      double *out);
void oracle_argmax_rows(const void *logits, int dtype, int64_t rows, int V, int32_t *out);
void oracle_accept(const void *target_logits, int dtype, const int32_t *target_ids,
                   const int32_t *tokens, const int32_t *parents, const int32_t *num_nodes,
                   int batch, int T, int V, int L, int32_t *accepted, int32_t *accepted_nodes,
                   int32_t *accept_len, int32_t *bonus, int32_t *target_argmax);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
int oracle_sample_row(const void *row, int dtype, int V, float tau, uint64_t seed, uint64_t offset,
                      int b, int i);
void oracle_accept_sample(const void *target_logits, int dtype, const int32_t *tokens,
                          const int32_t *parents, const int32_t *num_nodes, int batch, int T, int V,
                          int L, float tau, uint64_t seed, uint64_t offset, int32_t *accepted,
                          int32_t *accepted_nodes, int32_t *accept_len, int32_t *bonus,
                          int32_t *target_tokens);
void oracle_commit_kv(void *k_cache, void *v_cache, size_t row_bytes, const int64_t *kv_offsets,
                      const int32_t *prefix_lens, const int32_t *accept_len,
                      const int32_t *accepted_nodes, const int32_t *bonus, int batch, int L, int T,
                      int64_t total_rows, int32_t *new_prefix_lens, int32_t *next_roots);
uint64_t oracle_exp_fixed(float d);
double oracle_log64(double s);
void oracle_set_threads(int n);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t rnd32(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 16);
}

static float rnd_normal(void)
{
    float s = 0.0f;
    for (int k = 0; k < 12; ++k)
        s += (float)(rnd32() & 0xFFFF) / 65536.0f;
    return s - 6.0f;
}

static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16); /* truncation is enough for test inputs */
}

static int g_fail = 0;

#define CHECK(c, ...)                                                                       \
    do {                                                                                    \
        if (!(c)) {                                                                         \
            fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__);                  \
            fprintf(stderr, __VA_ARGS__);                                                   \
            fprintf(stderr, "\n");                                                          \
            g_fail = 1;                                                                     \
        }                                                                                   \
    } while (0)

/* Logits with the special values the numerics spec handles: ties (values
 * quantised to a coarse grid), NaN, +inf, -inf, and whole -inf rows. */
static void fill_logits(void *buf, int dtype, size_t n, int V, int special)
{
    for (size_t i = 0; i < n; ++i) {
        float x = rnd_normal() * 2.0f;
        if (special & 1)
            x = floorf(x * 2.0f) * 0.5f;
        uint32_t r = rnd32() % 97;
        if ((special & 2) && r == 0)
            x = NAN;
        else if ((special & 2) && r == 1)
            x = INFINITY;
        else if ((special & 2) && r == 2)
            x = -INFINITY;
        if ((special & 4) && (i / (size_t)V) % 3 == 1)
            x = -INFINITY; /* every third row has no finite value */
        if (dtype == 0)
            ((uint16_t *)buf)[i] = to_bf16(x);
        else
            ((float *)buf)[i] = x;
    }
}

static void check_tree(const int32_t *tokens, const int32_t *parents, const int32_t *depths,
                       int nn, int T, int L, const uint64_t *mask, int32_t root)
{
    CHECK(nn >= 1 && nn <= T, "num_nodes %d outside [1, %d]", nn, T);
    CHECK(tokens[0] == root && parents[0] == -1 && depths[0] == 0, "root row");
    int W = (T + 63) / 64;
    for (int i = 1; i < nn; ++i) {
        CHECK(parents[i] >= 0 && parents[i] < i, "node %d parent %d", i, parents[i]);
        if (parents[i] >= 0 && parents[i] < i)
            CHECK(depths[i] == depths[parents[i]] + 1 && depths[i] <= L, "node %d depth", i);
    }
    if (!mask)
        return;
    for (int i = 0; i < nn; ++i) {
        /* exactly the ancestors and the node itself */
        int cnt = 0;
        for (int j = 0; j < T; ++j)
            cnt += (int)((mask[(size_t)i * W + j / 64] >> (j % 64)) & 1u);
        CHECK(cnt == depths[i] + 1, "mask row %d has %d bits, depth %d", i, cnt, depths[i]);
        for (int a = i; a >= 0; a = parents[a])
            CHECK((mask[(size_t)i * W + a / 64] >> (a % 64)) & 1u, "mask row %d misses %d", i, a);
    }
}

static void run_build(int dtype, int B, int L, int V, int K, int N, float tau, int special)
{
    size_t es = dtype == 0 ? 2 : 4, n = (size_t)B * L * V;
    int T = N + 1, W = (T + 63) / 64;
    void *x = malloc(n * es);
    fill_logits(x, dtype, n, V, special);
    int32_t *roots = malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b)
        roots[b] = (int32_t)(rnd32() % (uint32_t)V);
    int32_t *tok = malloc(sizeof(int32_t) * B * T), *par = malloc(sizeof(int32_t) * B * T);
    int32_t *dep = malloc(sizeof(int32_t) * B * T), *nn = malloc(sizeof(int32_t) * B);
    float *sc = malloc(sizeof(float) * B * T);
    uint64_t *mask = malloc(sizeof(uint64_t) * (size_t)B * T * W);
    int32_t *ttok = malloc(sizeof(int32_t) * B * L * K), *st = malloc(sizeof(int32_t) * B);
    float *tlp = malloc(sizeof(float) * B * L * K), *rm = malloc(sizeof(float) * B * L);
    float *rl = malloc(sizeof(float) * B * L);
    uint64_t *rs = malloc(sizeof(uint64_t) * B * L);
    oracle_build(x, dtype, roots, B, L, V, K, N, tau, tok, par, dep, sc, nn, mask, ttok, tlp, st,
                 rm, rs, rl);
    for (int b = 0; b < B; ++b)
        check_tree(tok + (size_t)b * T, par + (size_t)b * T, dep + (size_t)b * T, nn[b], T, L,
                   mask + (size_t)b * T * W, roots[b]);
    /* the same rows one at a time, and the tree from the tables */
    int32_t *t1 = malloc(sizeof(int32_t) * K);
    float *l1 = malloc(sizeof(float) * K), m1, lse1;
    uint64_t S1;
    for (int r = 0; r < B * L; ++r) {
        oracle_row_topk((const char *)x + (size_t)r * V * es, dtype, V, K, tau, t1, l1, &m1, &S1,
                        &lse1);
        CHECK(memcmp(t1, ttok + (size_t)r * K, sizeof(int32_t) * K) == 0, "row %d top-K", r);
    }
    int n0 = oracle_tree(ttok, tlp, L, K, N, roots[0], tok, par, dep, sc);
    CHECK(n0 == nn[0], "tree of request 0: %d vs %d nodes", n0, nn[0]);
    oracle_mask(par, n0, T, mask);
    check_tree(tok, par, dep, n0, T, L, mask, roots[0]);
    free(t1); free(l1);
    free(x); free(roots); free(tok); free(par); free(dep); free(nn); free(sc); free(mask);
    free(ttok); free(st); free(tlp); free(rm); free(rl); free(rs);
}

/* Attention over caches of total_rows rows; request b's region starts at
 * offs[b]. Malformed requests (negative offset or prefix, region past the
 * end, offsets near INT64_MAX) must give zero rows without touching memory
 * outside the caches. */
static void run_attn(int dtype, int B, int T, int Hq, int Hkv, int D)
{
    size_t es = dtype == 0 ? 2 : 4;
    int W = (T + 63) / 64;
    int32_t *P = malloc(sizeof(int32_t) * B), *nn = malloc(sizeof(int32_t) * B);
    int64_t *offs = malloc(sizeof(int64_t) * B), total = 0;
    for (int b = 0; b < B; ++b) {
        P[b] = (int32_t)(b % 3 == 0 ? 0 : rnd32() % 150);
        nn[b] = 1 + (int32_t)(rnd32() % (uint32_t)T);
        offs[b] = total;
        total += P[b] + T;
    }
    size_t qn = (size_t)B * T * Hq * D, kn = (size_t)total * Hkv * D;
    void *q = malloc(qn * es), *k = malloc(kn * es), *v = malloc(kn * es);
    fill_logits(q, dtype, qn, D, 0);
    fill_logits(k, dtype, kn, D, 0);
    fill_logits(v, dtype, kn, D, 0);
    uint64_t *mask = calloc((size_t)B * T * W, sizeof(uint64_t));
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < T; ++i) /* a chain: node i's ancestors are 0..i */
            for (int j = 0; j <= i; ++j)
                mask[((size_t)b * T + i) * W + j / 64] |= 1ull << (j % 64);
    int nsel = B * T * Hq;
    int32_t *sel = malloc(sizeof(int32_t) * 3 * nsel);
    for (int s = 0; s < nsel; ++s) {
        sel[3 * s] = s / (T * Hq);
        sel[3 * s + 1] = (s / Hq) % T;
        sel[3 * s + 2] = s % Hq;
    }
    double *out = malloc(sizeof(double) * (size_t)nsel * D);
    oracle_attn_rows(q, k, v, dtype, offs, P, nn, mask, T, Hq, Hkv, D, total,
                     1.0 / sqrt((double)D), sel, nsel, out);
    for (int s = 0; s < nsel; ++s) {
        int b = sel[3 * s], i = sel[3 * s + 1];
        for (int d = 0; d < D; ++d)
            CHECK(isfinite(out[(size_t)s * D + d]), "attention row %d not finite", s);
        if (i >= nn[b])
            for (int d = 0; d < D; ++d)
                CHECK(out[(size_t)s * D + d] == 0.0, "padding row %d not zero", s);
    }
    const int64_t bad_offs[] = {-1, total - P[B - 1] - T + 1, INT64_MAX - 3, INT64_MIN + 3};
    for (int c = 0; c < 4; ++c) {
        int64_t keep = offs[B - 1];
        offs[B - 1] = bad_offs[c];
        oracle_attn_rows(q, k, v, dtype, offs, P, nn, mask, T, Hq, Hkv, D, total, 0.125, sel,
                         nsel, out);
        for (int s = 0; s < nsel; ++s)
            if (sel[3 * s] == B - 1)
                for (int d = 0; d < D; ++d)
                    CHECK(out[(size_t)s * D + d] == 0.0, "malformed request row %d not zero", s);
        offs[B - 1] = keep;
    }
    int32_t keepP = P[0];
    P[0] = -5;
    oracle_attn_rows(q, k, v, dtype, offs, P, nn, mask, T, Hq, Hkv, D, total, 0.125, sel, nsel,
                     out);
    P[0] = keepP;
    free(P); free(nn); free(offs); free(q); free(k); free(v); free(mask); free(sel); free(out);
}

/* Trees for the walk: node i's parent drawn among 0..i-1, tokens small so
 * that siblings repeat tokens (the walk takes the first matching child). */
static void random_tree(int32_t *tok, int32_t *par, int T, int V)
{
    tok[0] = 0;
    par[0] = -1;
    for (int i = 1; i < T; ++i) {
        par[i] = (int32_t)(rnd32() % (uint32_t)i);
        tok[i] = (int32_t)(rnd32() % (uint32_t)(V < 4 ? V : 4));
    }
}

static void run_accept(int dtype, int B, int T, int V, int L, int sample)
{
    size_t es = dtype == 0 ? 2 : 4;
    void *tl = malloc((size_t)B * T * V * es);
    fill_logits(tl, dtype, (size_t)B * T * V, V, 2 | 4);
    int32_t *tok = malloc(sizeof(int32_t) * B * T), *par = malloc(sizeof(int32_t) * B * T);
    int32_t *nn = malloc(sizeof(int32_t) * B), *ids = malloc(sizeof(int32_t) * B * T);
    for (int b = 0; b < B; ++b) {
        random_tree(tok + (size_t)b * T, par + (size_t)b * T, T, V);
        nn[b] = b % 2 ? T : 1 + (int32_t)(rnd32() % (uint32_t)T);
    }
    for (int r = 0; r < B * T; ++r)
        ids[r] = (int32_t)(rnd32() % 4u);
    int32_t *acc = malloc(sizeof(int32_t) * B * L), *accn = malloc(sizeof(int32_t) * B * L);
    int32_t *alen = malloc(sizeof(int32_t) * B), *bonus = malloc(sizeof(int32_t) * B);
    int32_t *tgt = malloc(sizeof(int32_t) * B * T);
    for (int pass = 0; pass < 2; ++pass) {
        if (sample)
            oracle_accept_sample(tl, dtype, tok, par, nn, B, T, V, L, pass ? 0.5f : 1.0f,
                                 0x1234567890ull, (uint64_t)pass * 77, acc, accn, alen, bonus,
                                 pass ? NULL : tgt);
        else
            oracle_accept(pass ? NULL : tl, dtype, pass ? ids : NULL, tok, par, nn, B, T, V, L,
                          acc, accn, alen, bonus, pass ? NULL : tgt);
        for (int b = 0; b < B; ++b) {
            CHECK(alen[b] >= 0 && alen[b] <= L, "accept_len %d", alen[b]);
            int cur = 0;
            for (int k = 0; k < alen[b]; ++k) {
                int c = accn[(size_t)b * L + k];
                CHECK(c >= 1 && c < nn[b] && par[(size_t)b * T + c] == cur, "walk step %d", k);
                if (c < 1 || c >= nn[b])
                    break;
                cur = c;
            }
        }
    }
    int32_t *am = malloc(sizeof(int32_t) * B * T);
    oracle_argmax_rows(tl, dtype, (int64_t)B * T, V, am);
    for (int r = 0; r < B * T; ++r)
        CHECK(am[r] >= 0 && am[r] < V, "argmax %d", am[r]);
    for (int r = 0; r < 4 && r < B * T; ++r) {
        int s = oracle_sample_row((const char *)tl + (size_t)r * V * es, dtype, V, 0.7f, 99, 3,
                                  r, 0);
        CHECK(s >= 0 && s < V, "sample %d", s);
    }
    free(tl); free(tok); free(par); free(nn); free(ids); free(acc); free(accn); free(alen);
    free(bonus); free(tgt); free(am);
}

static void run_commit(int B, int L, int T, size_t row_bytes)
{
    int32_t *P = malloc(sizeof(int32_t) * B), *alen = malloc(sizeof(int32_t) * B);
    int32_t *an = malloc(sizeof(int32_t) * B * L), *bonus = malloc(sizeof(int32_t) * B);
    int32_t *np = malloc(sizeof(int32_t) * B), *nr = malloc(sizeof(int32_t) * B);
    int64_t *offs = malloc(sizeof(int64_t) * B), total = 0;
    for (int b = 0; b < B; ++b) {
        P[b] = (int32_t)(rnd32() % 40);
        offs[b] = total;
        total += P[b] + T + 3;
        alen[b] = (int32_t)(rnd32() % (uint32_t)(L + 1));
        if (alen[b] > T - 1)
            alen[b] = T - 1;
        for (int k = 0; k < L; ++k)
            an[(size_t)b * L + k] = 1 + (int32_t)(rnd32() % (uint32_t)(T - 1 > 0 ? T - 1 : 1));
        bonus[b] = b;
    }
    /* malformed requests, one per kind */
    if (B >= 7) {
        alen[1] = L + 1;
        alen[2] = -1;
        an[(size_t)3 * L] = T;
        alen[3] = alen[3] > 0 ? alen[3] : 1;
        offs[4] = -2;
        P[5] = -1;
        offs[6] = INT64_MAX - 2;
    }
    unsigned char *kc = malloc((size_t)total * row_bytes), *vc = malloc((size_t)total * row_bytes);
    for (size_t i = 0; i < (size_t)total * row_bytes; ++i) {
        kc[i] = (unsigned char)rnd32();
        vc[i] = (unsigned char)rnd32();
    }
    oracle_commit_kv(kc, vc, row_bytes, offs, P, alen, an, bonus, B, L, T, total, np, nr);
    for (int b = 0; b < B; ++b)
        CHECK(np[b] == -1 || np[b] == P[b] + 1 + alen[b], "new prefix %d", np[b]);
    oracle_commit_kv(kc, vc, row_bytes, offs, P, alen, an, bonus, B, L, T, total, np, NULL);
    free(P); free(alen); free(an); free(bonus); free(np); free(nr); free(offs); free(kc); free(vc);
}

int main(void)
{
    for (int threads = 1; threads <= 3; threads += 2) {
        oracle_set_threads(threads);
        for (int dt = 0; dt < 2; ++dt) {
            run_build(dt, 2, 3, 17, 4, 20, 1.0f, 0);
            run_build(dt, 1, 1, 1, 1, 1, 1.0f, 0);          /* smallest everything */
            run_build(dt, 3, 4, 64, 8, 200, 0.7f, 1 | 2);   /* ties, NaN, +-inf */
            run_build(dt, 2, 5, 40, 40, 1024, 1.0f, 1);     /* K = V, budget above the tree */
            run_build(dt, 3, 6, 50, 5, 130, 0.0f, 1 | 4);   /* argmax mode, -inf rows */
            run_build(dt, 1, 32, 300, 16, 1024, 1.3f, 1);   /* deepest block, largest budget */
            run_attn(dt, 4, 70, 8, 2, 32);                  /* mask over two words */
            run_attn(dt, 2, 1, 4, 4, 64);
            run_accept(dt, 5, 33, 50, 6, 0);
            run_accept(dt, 5, 33, 50, 6, 1);
            run_accept(dt, 2, 1, 1, 1, 1);                  /* V = 1, T = 1 */
        }
        run_commit(9, 4, 12, 64);
        run_commit(1, 1, 1, 16);
    }
    for (int i = -200; i <= 0; ++i)
        (void)oracle_exp_fixed((float)i * 0.37f);
    (void)oracle_exp_fixed(-INFINITY);
    (void)oracle_log64(1.0);
    (void)oracle_log64(3.0e12);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    oracle_philox4x32_10(ctr, key, o);
    if (g_fail)
        return 1;
    printf("oracle driver: all paths ran clean\n");
    return 0;
}
