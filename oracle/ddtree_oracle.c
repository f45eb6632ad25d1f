/*
 * CPU oracle for the DDTree per-round hot path.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers. The GPU library never
 * includes, links or calls anything in this directory, and this file shares
 * no code, header or constant generator with it.
 *
 * Source page (cited below as [BDDT <section>]):
 *   "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
 *   (Ringel, Romano) -- source-linked summary page of the paper.
 *
 * What is computed, per decoding round:
 *   1. per-position log-probabilities of the drafter's marginals q_i and
 *      their top-K candidates                        [BDDT §3, §4.1, App. A]
 *   2. the best-first tree: B pops of a priority queue ordered by cumulative
 *      log-probability, each pop pushing the popped prefix's next sibling
 *      and its best child                              [BDDT §4.3, App. A]
 *   3. the ancestor-only attention mask                [BDDT Abstract, §4.1]
 *   4. tree attention of every node over the prefix KV and its ancestors,
 *      naive fp64                                      [BDDT Abstract, App. B]
 *   5. the target's greedy decoding rule (argmax) and the tree walk that
 *      accepts the matched path and emits the bonus token  [BDDT §4.1]
 *   6. at target temperature > 0, the target's sample per node (Philox
 *      counter-based uniforms) and the same walk           [BDDT §4.1]
 *   7. the KV compaction of the accepted path and the bonus hand-off
 *                                                          [BDDT §4.1]
 *
 * The pages fix no arithmetic for step 1. Because the tree order compares
 * sums of log-probabilities taken at different depths, both implementations
 * must produce the same bits, so step 1 follows an explicit numerics
 * specification (every operation an IEEE-754 basic operation or fmaf):
 *
 *   x_v   = fp32(logit_v * fp32(1/tau))            (tau > 0)
 *         = logit_v                                (tau == 0, argmax mode)
 *           NaN and +inf become -inf (status bit 0)
 *   m     = max_v x_v            (all -inf: status bit 1, every lp = -inf)
 *   d_v   = fp32(x_v - m)        (tau > 0)
 *         = 0 if x_v == m else -inf                (tau == 0)
 *   u_v   = rint(2^44 * E(d_v))  E: fp32 exponential below (exp_fixed)
 *   S     = sum_v u_v            exact in uint64 (V <= 2^19), order-free
 *   lse   = fp32(LOG64(S * 2^-44))   LOG64: fp64 logarithm below
 *   lp_k  = fp32(d_{v_k} - lse)  for the K tokens ranked by (x desc, id asc)
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp (no fast-math).
 *
 * Threads: one by default. oracle_set_threads(n) lets the batch-level
 * functions spread independent units over n OpenMP threads -- drafter rows
 * and then requests (build), query rows (attention), target rows and then
 * requests (accept) -- each unit computed by the same serial code, so the
 * results do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ODT_BF16 0
#define ODT_F32 1

static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n > 0 ? n : 1; }

int oracle_get_threads(void) { return g_threads; }

static float load_value(const void *base, int dtype, size_t idx)
{
    if (dtype == ODT_BF16) {
        /* bfloat16 is the upper half of an IEEE fp32 word: widening is exact */
        uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    return ((const float *)base)[idx];
}

/* ------------------------------------------------------------------------ */
/* fp32 exponential in 2^44 fixed point.                                     */
/*                                                                          */
/* e^d = 2^t with t = d*log2(e); t = n + f with n = rint(t), |f| <= 1/2;     */
/* 2^f by its Taylor series truncated after degree 5, coefficients           */
/* (ln 2)^k / k! rounded to fp32, evaluated by Horner with fused multiply-   */
/* adds; the result scaled by 2^(n+44) and rounded to the nearest integer.   */
/* t is clamped at -64, where the result is 0 after rounding (and which also */
/* maps d = -inf). The maximal element (d = 0) gives exactly 2^44.           */
/* ------------------------------------------------------------------------ */
uint64_t oracle_exp_fixed(float d)
{
    const float log2e = 0x1.715476p+0f;   /* fp32(1/ln 2) */
    const float c0 = 1.0f;
    const float c1 = 0x1.62e430p-1f;      /* fp32(ln2)        */
    const float c2 = 0x1.ebfbe0p-3f;      /* fp32(ln2^2/2)    */
    const float c3 = 0x1.c6b08ep-5f;      /* fp32(ln2^3/6)    */
    const float c4 = 0x1.3b2ab6p-7f;      /* fp32(ln2^4/24)   */
    const float c5 = 0x1.5d87fep-10f;     /* fp32(ln2^5/120)  */
    float t = d * log2e;
    t = fmaxf(t, -64.0f);
    float n = rintf(t);
    float f = t - n;
    float p = c5;
    p = fmaf(p, f, c4);
    p = fmaf(p, f, c3);
    p = fmaf(p, f, c2);
    p = fmaf(p, f, c1);
    p = fmaf(p, f, c0);
    float e = ldexpf(p, (int)n + 44);
    return (uint64_t)rintf(e);
}

/* ------------------------------------------------------------------------ */
/* fp64 natural logarithm for s > 0.                                         */
/* s = mant * 2^k with mant in [sqrt(1/2), sqrt(2));                         */
/* ln s = k ln2 + 2 atanh(z), z = (mant-1)/(mant+1), |z| < 0.1716;           */
/* atanh(z) = z * sum_{j=0..11} w^j/(2j+1), w = z^2, by Horner in w.         */
/* The dropped tail is below 1e-18 relative.                                 */
/* ------------------------------------------------------------------------ */
double oracle_log64(double s)
{
    const double ln2 = 0x1.62e42fefa39efp-1;
    const double rsqrt2 = 0x1.6a09e667f3bcdp-1;
    int k;
    double mant = frexp(s, &k); /* s = mant * 2^k, mant in [0.5, 1) */
    if (mant < rsqrt2) {
        mant = mant * 2.0;
        k = k - 1;
    }
    double z = (mant - 1.0) / (mant + 1.0);
    double w = z * z;
    double a = 1.0 / 23.0;
    a = a * w + 1.0 / 21.0;
    a = a * w + 1.0 / 19.0;
    a = a * w + 1.0 / 17.0;
    a = a * w + 1.0 / 15.0;
    a = a * w + 1.0 / 13.0;
    a = a * w + 1.0 / 11.0;
    a = a * w + 1.0 / 9.0;
    a = a * w + 1.0 / 7.0;
    a = a * w + 1.0 / 5.0;
    a = a * w + 1.0 / 3.0;
    a = a * w + 1.0;
    double head = (double)k * ln2;
    double tail = (2.0 * z) * a;
    return head + tail;
}

/* S * 2^-44 as a double: the high and low 32-bit halves are exact doubles,  */
/* so the single rounding is that of the final addition.                     */
static double fixed_to_double(uint64_t S)
{
    double hi = (double)(uint32_t)(S >> 32) * 4294967296.0;
    double lo = (double)(uint32_t)(S & 0xffffffffu);
    return (hi + lo) * 0x1p-44;
}

/* ------------------------------------------------------------------------ */
/* Step 1: log-softmax of one drafter row and its top-K       [BDDT §3, §4.3]*/
/* ------------------------------------------------------------------------ */
static float sanitized(const void *row, int dtype, size_t v, float tau, float inv_tau,
                       int *flags)
{
    float x = load_value(row, dtype, v);
    if (tau > 0.0f)
        x = x * inv_tau;
    if (isnan(x) || x == INFINITY) {
        *flags |= 1;
        x = -INFINITY;
    }
    return x;
}

static float diff_from_max(float x, float m, float tau)
{
    if (tau > 0.0f)
        return x - m;
    return (x == m) ? 0.0f : -INFINITY;
}

/*
 * One row of V logits -> top-K token ids and log-probabilities.
 * Ranking: x descending, token id ascending on ties (x after temperature
 * scaling and NaN/+inf replacement). Returns the status bits of the row.
 * Diagnostics (row max, fixed-point sum, lse) are written when non-NULL.
 */
int oracle_row_topk(const void *row, int dtype, int V, int K, float tau, int32_t *topk_tok,
                    float *topk_lp, float *out_m, uint64_t *out_S, float *out_lse)
{
    int flags = 0;
    float inv_tau = (tau > 0.0f) ? 1.0f / tau : 1.0f;

    float m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        float x = sanitized(row, dtype, (size_t)v, tau, inv_tau, &flags);
        if (x > m)
            m = x;
    }

    /* top-K by insertion into a list kept sorted by (x desc, id asc) */
    float *bx = (float *)malloc(sizeof(float) * (size_t)K);
    int32_t *bv = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    int cnt = 0;
    int dummy = 0;
    for (int v = 0; v < V; ++v) {
        float x = sanitized(row, dtype, (size_t)v, tau, inv_tau, &dummy);
        if (cnt == K && !(x > bx[K - 1]))
            continue; /* ties with the K-th keep the smaller id already held */
        int pos = (cnt < K) ? cnt : K - 1;
        while (pos > 0 && bx[pos - 1] < x) {
            if (pos < K) {
                bx[pos] = bx[pos - 1];
                bv[pos] = bv[pos - 1];
            }
            --pos;
        }
        bx[pos] = x;
        bv[pos] = v;
        if (cnt < K)
            ++cnt;
    }

    uint64_t S = 0;
    float lse = INFINITY;
    if (m == -INFINITY) {
        flags |= 2;
        for (int k = 0; k < K; ++k) {
            topk_tok[k] = bv[k];
            topk_lp[k] = -INFINITY;
        }
    } else {
        for (int v = 0; v < V; ++v) {
            float x = sanitized(row, dtype, (size_t)v, tau, inv_tau, &dummy);
            S += oracle_exp_fixed(diff_from_max(x, m, tau));
        }
        lse = (float)oracle_log64(fixed_to_double(S));
        for (int k = 0; k < K; ++k) {
            topk_tok[k] = bv[k];
            topk_lp[k] = diff_from_max(bx[k], m, tau) - lse;
        }
    }
    if (out_m)
        *out_m = m;
    if (out_S)
        *out_S = S;
    if (out_lse)
        *out_lse = lse;
    free(bx);
    free(bv);
    return flags;
}

/* ------------------------------------------------------------------------ */
/* Step 2: best-first tree under node budget N       [BDDT §4.2, §4.3, App. A]*/
/*                                                                          */
/* A candidate is (parent node, depth, rank): the rank-th best token of      */
/* position `depth` appended to the parent's prefix. Its score is the fp32   */
/* cumulative log-probability, accumulated from the root: score(parent)+lp.  */
/* Order: score descending, then depth, parent node index, rank ascending.   */
/* (At most one candidate per parent is pending at a time, so the rank field */
/* never decides; it is kept so that the order is total by construction.)    */
/* Each pop becomes the next node; it pushes its next sibling (same parent,  */
/* rank+1) and its best child (depth+1, rank 0). The priority queue is an    */
/* unsorted array searched linearly for its best element.                    */
/* ------------------------------------------------------------------------ */
typedef struct {
    float score;
    int depth, parent, rank;
} cand_t;

static int cand_better(const cand_t *a, const cand_t *b)
{
    if (a->score != b->score)
        return a->score > b->score;
    if (a->depth != b->depth)
        return a->depth < b->depth;
    if (a->parent != b->parent)
        return a->parent < b->parent;
    return a->rank < b->rank;
}

/* Arrays have T = N+1 rows; returns num_nodes (root included). */
int oracle_tree(const int32_t *topk_tok, const float *topk_lp, int L, int K, int N,
                int32_t root_token, int32_t *tokens, int32_t *parents, int32_t *depths,
                float *scores)
{
    int T = N + 1;
    for (int i = 0; i < T; ++i) {
        tokens[i] = -1;
        parents[i] = -1;
        depths[i] = -1;
        scores[i] = -INFINITY;
    }
    tokens[0] = root_token;
    depths[0] = 0;
    scores[0] = 0.0f;

    cand_t *pq = (cand_t *)malloc(sizeof(cand_t) * (size_t)(2 * N + 2));
    int npq = 0;
    if (L >= 1 && K >= 1) {
        cand_t c = {scores[0] + topk_lp[0], 1, 0, 0};
        pq[npq++] = c;
    }
    int n = 1;
    while (n <= N && npq > 0) {
        int best = 0;
        for (int j = 1; j < npq; ++j)
            if (cand_better(&pq[j], &pq[best]))
                best = j;
        cand_t c = pq[best];
        pq[best] = pq[--npq];

        tokens[n] = topk_tok[(size_t)(c.depth - 1) * K + c.rank];
        parents[n] = c.parent;
        depths[n] = c.depth;
        scores[n] = c.score;

        if (c.rank + 1 < K) {
            cand_t sib = {scores[c.parent] + topk_lp[(size_t)(c.depth - 1) * K + c.rank + 1],
                          c.depth, c.parent, c.rank + 1};
            pq[npq++] = sib;
        }
        if (c.depth + 1 <= L) {
            cand_t child = {c.score + topk_lp[(size_t)c.depth * K], c.depth + 1, n, 0};
            pq[npq++] = child;
        }
        ++n;
    }
    free(pq);
    return n;
}

/* ------------------------------------------------------------------------ */
/* Step 3: ancestor-only mask                           [BDDT Abstract, §4.1]*/
/* Row i has bit j set (word j/64, bit j%64) iff j is i or an ancestor of i. */
/* Rows at or beyond num_nodes are zero.                                     */
/* ------------------------------------------------------------------------ */
void oracle_mask(const int32_t *parents, int num_nodes, int T, uint64_t *mask)
{
    int W = (T + 63) / 64;
    memset(mask, 0, sizeof(uint64_t) * (size_t)T * (size_t)W);
    for (int i = 0; i < num_nodes; ++i) {
        int j = i;
        while (j >= 0) {
            mask[(size_t)i * W + (size_t)(j / 64)] |= 1ull << (j % 64);
            j = parents[j];
        }
    }
}

/* Steps 1-3 for a batch. logits [batch, L, V]; tree arrays [batch, N+1];
 * mask [batch, N+1, W] (NULL skips it); topk [batch, L, K]; status [batch];
 * row diagnostics [batch, L] (each NULL to skip). */
void oracle_build(const void *logits, int dtype, const int32_t *root_tokens, int batch, int L,
                  int V, int K, int N, float tau, int32_t *tokens, int32_t *parents,
                  int32_t *depths, float *scores, int32_t *num_nodes, uint64_t *mask,
                  int32_t *topk_tok, float *topk_lp, int32_t *status, float *row_m,
                  uint64_t *row_S, float *row_lse)
{
    int T = N + 1;
    int W = (T + 63) / 64;
    size_t elem = (dtype == ODT_BF16) ? 2 : 4;
    int rows = batch * L;
    int *row_flags = (int *)malloc(sizeof(int) * (size_t)(rows > 0 ? rows : 1));
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int r = 0; r < rows; ++r) {
        const char *row = (const char *)logits + (size_t)r * (size_t)V * elem;
        row_flags[r] = oracle_row_topk(row, dtype, V, K, tau, topk_tok + (size_t)r * K,
                                       topk_lp + (size_t)r * K, row_m ? row_m + r : NULL,
                                       row_S ? row_S + r : NULL, row_lse ? row_lse + r : NULL);
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int b = 0; b < batch; ++b) {
        int flags = 0;
        for (int i = 0; i < L; ++i)
            flags |= row_flags[b * L + i];
        if (status)
            status[b] = flags;
        size_t o = (size_t)b * T;
        num_nodes[b] = oracle_tree(topk_tok + (size_t)b * L * K, topk_lp + (size_t)b * L * K, L,
                                   K, N, root_tokens[b], tokens + o, parents + o, depths + o,
                                   scores + o);
        if (mask)
            oracle_mask(parents + o, num_nodes[b], T, mask + o * W);
    }
    free(row_flags);
}

/* ------------------------------------------------------------------------ */
/* Step 4: tree attention, naive fp64               [BDDT Abstract, App. B]  */
/*                                                                          */
/* q, out [batch, T, Hq, D]; k, v [rows, Hkv, D] with request b's rows at    */
/* kv_offsets[b]: P_b prefix rows, then T tree rows in node order.           */
/* Query (b, i, h) attends to every prefix row and to tree rows j whose mask */
/* bit (i, j) is set; q-head h reads kv-head h / (Hq/Hkv). Rows i at or      */
/* beyond num_nodes[b] are zero, and so are all rows of a request whose K/V  */
/* rows kv_offsets[b] .. kv_offsets[b] + P_b + T do not lie inside the      */
/* total_rows rows of the caches. Only the (b, i, h) triples in sel are     */
/* computed, into out[nsel, D].                                              */
/* ------------------------------------------------------------------------ */
void oracle_attn_rows(const void *q, const void *k, const void *v, int dtype,
                      const int64_t *kv_offsets, const int32_t *prefix_lens,
                      const int32_t *num_nodes, const uint64_t *mask, int T, int Hq, int Hkv,
                      int D, int64_t total_rows, double scale, const int32_t *sel, int nsel,
                      double *out)
{
    int g = Hq / Hkv;
    int W = (T + 63) / 64;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int s = 0; s < nsel; ++s) {
        int b = sel[3 * s], i = sel[3 * s + 1], h = sel[3 * s + 2];
        double *o = out + (size_t)s * D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        if (i >= num_nodes[b])
            continue;
        /* written so that no sum can overflow */
        if (kv_offsets[b] < 0 || prefix_lens[b] < 0 ||
            kv_offsets[b] > total_rows - (int64_t)prefix_lens[b] - T)
            continue;
        int P = prefix_lens[b];
        int hk = h / g;
        size_t qbase = (((size_t)b * T + i) * Hq + h) * D;
        const uint64_t *mrow = mask + ((size_t)b * T + i) * W;
        int nkeys = P + T;
        double *sc = (double *)malloc(sizeof(double) * (size_t)nkeys);
        char *ok = (char *)malloc((size_t)nkeys);
        double mx = -INFINITY;
        for (int j = 0; j < nkeys; ++j) {
            if (j < P) {
                ok[j] = 1;
            } else {
                int t = j - P;
                ok[j] = (char)((mrow[t / 64] >> (t % 64)) & 1u);
            }
            if (!ok[j])
                continue;
            size_t kbase = (((size_t)kv_offsets[b] + j) * Hkv + hk) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += (double)load_value(q, dtype, qbase + d) *
                       (double)load_value(k, dtype, kbase + d);
            sc[j] = scale * dot;
            if (sc[j] > mx)
                mx = sc[j];
        }
        double den = 0.0;
        for (int j = 0; j < nkeys; ++j) {
            if (!ok[j])
                continue;
            double p = exp(sc[j] - mx);
            den += p;
            size_t vbase = (((size_t)kv_offsets[b] + j) * Hkv + hk) * D;
            for (int d = 0; d < D; ++d)
                o[d] += p * (double)load_value(v, dtype, vbase + d);
        }
        if (den > 0.0)
            for (int d = 0; d < D; ++d)
                o[d] /= den;
        free(sc);
        free(ok);
    }
}

/* ------------------------------------------------------------------------ */
/* Step 5a: the target's greedy decoding rule                    [BDDT §4.1] */
/* First index of the maximum; NaN counts as -inf; an all -inf row gives 0.  */
/* ------------------------------------------------------------------------ */
void oracle_argmax_rows(const void *logits, int dtype, int64_t rows, int V, int32_t *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        float best = -INFINITY;
        int idx = 0;
        for (int v = 0; v < V; ++v) {
            float x = load_value(logits, dtype, (size_t)r * V + v);
            if (x > best) {
                best = x;
                idx = v;
            }
        }
        out[r] = idx;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 5b: tree walk with the target's tokens                   [BDDT §4.1] */
/*                                                                          */
/* From the root, follow the child whose token equals the target's token at */
/* the current node; the matched path is accepted and the first unmatched   */
/* target token is the bonus. tgt[i] is the target's token after node i.    */
/* accepted / accepted_nodes have L slots, padded with -1. A walk that has  */
/* accepted L nodes stops there (a depth-L node has no children).           */
/* ------------------------------------------------------------------------ */
void oracle_walk(const int32_t *tokens, const int32_t *parents, int num_nodes, const int32_t *tgt,
                 int L, int32_t *accepted, int32_t *accepted_nodes, int32_t *accept_len,
                 int32_t *bonus)
{
    for (int k = 0; k < L; ++k) {
        accepted[k] = -1;
        accepted_nodes[k] = -1;
    }
    int cur = 0, len = 0;
    for (;;) {
        int y = tgt[cur];
        int next = -1;
        for (int c = 1; c < num_nodes; ++c) {
            if (parents[c] == cur && tokens[c] == y) {
                next = c;
                break;
            }
        }
        if (next < 0 || len >= L) {
            *bonus = y;
            break;
        }
        accepted[len] = y;
        accepted_nodes[len] = next;
        ++len;
        cur = next;
    }
    *accept_len = len;
}

/* Steps 5a+5b for a batch: target logits [batch, T, V] (or target ids
 * [batch, T] when logits is NULL); tree arrays [batch, T]. Rows at or beyond
 * num_nodes[b] get argmax -1. */
void oracle_accept(const void *target_logits, int dtype, const int32_t *target_ids,
                   const int32_t *tokens, const int32_t *parents, const int32_t *num_nodes,
                   int batch, int T, int V, int L, int32_t *accepted, int32_t *accepted_nodes,
                   int32_t *accept_len, int32_t *bonus, int32_t *target_argmax)
{
    size_t elem = (dtype == ODT_BF16) ? 2 : 4;
    int32_t *tgt = (int32_t *)malloc(sizeof(int32_t) * (size_t)batch * (size_t)T);
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int64_t r = 0; r < (int64_t)batch * T; ++r) {
        int b = (int)(r / T), i = (int)(r % T);
        if (i >= num_nodes[b]) {
            tgt[r] = -1;
        } else if (target_logits) {
            const char *row = (const char *)target_logits + (size_t)r * (size_t)V * elem;
            oracle_argmax_rows(row, dtype, 1, V, &tgt[r]);
        } else {
            tgt[r] = target_ids[r];
        }
        if (target_argmax)
            target_argmax[r] = tgt[r];
    }
    for (int b = 0; b < batch; ++b) {
        size_t o = (size_t)b * T;
        oracle_walk(tokens + o, parents + o, num_nodes[b], tgt + o, L, accepted + (size_t)b * L,
                    accepted_nodes + (size_t)b * L, accept_len + b, bonus + b);
    }
    free(tgt);
}

/* ------------------------------------------------------------------------ */
/* Next step: acceptance at target temperature tau_t > 0         [BDDT §4.1] */
/*                                                                          */
/* The walk is the same; the target's token after node i is a sample of     */
/* softmax(logits_i / tau_t) instead of its argmax. The sample is exact and */
/* reproducible: the weights are the fixed-point terms u_v of the numerics  */
/* spec (x_v = fp32(logit_v * fp32(1/tau_t)), NaN / +inf -> -inf, m = max,  */
/* u_v = rint(2^44 E(x_v - m)), S = sum u_v), a 64-bit uniform r comes from */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as  */
/* easy as 1, 2, 3", SC 2011) with key (seed_lo, seed_hi) and counter       */
/* (i, b, offset_lo, offset_hi), r = word1 * 2^32 + word0, and the token is */
/* the first v whose running sum of u exceeds theta = floor(r * S / 2^64).  */
/* Token v is then drawn with probability u_v / S. A row without a finite   */
/* value (S = 0) gives token 0.                                             */
/*                                                                          */
/* Parity unpinned for the draw's convention: the pages fix no generator,   */
/* and the word order of r, the counter layout and the strict "exceeds"     */
/* are this implementation's choices. The pins fix the law of the draw      */
/* (chi-square against softmax, exact special cases), Philox itself (the    */
/* published known-answer vectors) and the counter's independence; the same */
/* convention changed on both sides would still pass them.                  */
/* ------------------------------------------------------------------------ */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k[0];
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k[1];
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
}

/* Philox4x32 with 10 rounds: the key is bumped by the Weyl constants between
 * rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        philox_round(c, k);
    }
    for (int j = 0; j < 4; ++j)
        out[j] = c[j];
}

/* The sampled token of one row (see above). */
int oracle_sample_row(const void *row, int dtype, int V, float tau, uint64_t seed, uint64_t offset,
                      int b, int i)
{
    const float inv_tau = 1.0f / tau;
    int flags = 0;
    float m = -INFINITY;
    for (int v = 0; v < V; ++v) {
        float x = sanitized(row, dtype, (size_t)v, tau, inv_tau, &flags);
        if (x > m)
            m = x;
    }
    if (m == -INFINITY)
        return 0;
    uint64_t S = 0;
    for (int v = 0; v < V; ++v)
        S += oracle_exp_fixed(sanitized(row, dtype, (size_t)v, tau, inv_tau, &flags) - m);
    const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)b, (uint32_t)offset, (uint32_t)(offset >> 32)};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    const uint64_t r = ((uint64_t)w[1] << 32) | w[0];
    const uint64_t theta = (uint64_t)(((unsigned __int128)r * S) >> 64);
    uint64_t run = 0;
    for (int v = 0; v < V; ++v) {
        run += oracle_exp_fixed(sanitized(row, dtype, (size_t)v, tau, inv_tau, &flags) - m);
        if (run > theta)
            return v;
    }
    return V - 1; /* not reached: run ends at S > theta */
}

/* Sampled target tokens and the walk for a batch; target_tokens [batch, T]
 * gets -1 for rows at or beyond num_nodes[b]. */
void oracle_accept_sample(const void *target_logits, int dtype, const int32_t *tokens,
                          const int32_t *parents, const int32_t *num_nodes, int batch, int T, int V,
                          int L, float tau, uint64_t seed, uint64_t offset, int32_t *accepted,
                          int32_t *accepted_nodes, int32_t *accept_len, int32_t *bonus,
                          int32_t *target_tokens)
{
    size_t elem = (dtype == ODT_BF16) ? 2 : 4;
    int32_t *tgt = (int32_t *)malloc(sizeof(int32_t) * (size_t)batch * (size_t)T);
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
    for (int64_t r = 0; r < (int64_t)batch * T; ++r) {
        int b = (int)(r / T), i = (int)(r % T);
        if (i >= num_nodes[b]) {
            tgt[r] = -1;
        } else {
            const char *row = (const char *)target_logits + (size_t)r * (size_t)V * elem;
            tgt[r] = oracle_sample_row(row, dtype, V, tau, seed, offset, b, i);
        }
        if (target_tokens)
            target_tokens[r] = tgt[r];
    }
    for (int b = 0; b < batch; ++b) {
        size_t o = (size_t)b * T;
        oracle_walk(tokens + o, parents + o, num_nodes[b], tgt + o, L, accepted + (size_t)b * L,
                    accepted_nodes + (size_t)b * L, accept_len + b, bonus + b);
    }
    free(tgt);
}

/* ------------------------------------------------------------------------ */
/* KV compaction after the walk, and the bonus hand-off            [BDDT §4.1] */
/*                                                                          */
/* Request b's K/V region starts at row kv_offsets[b]; after the verify its */
/* prefix holds rows [0, P) and the tree rows follow in node order (node i  */
/* at row P + i). The sequence the round commits is the prefix, the root    */
/* (node 0, already at row P) and the accepted nodes a_0 .. a_{n-1}: their  */
/* rows move to P + 1 .. P + n. Every move reads the rows as they were      */
/* before the first move (a source may be another move's destination). The  */
/* new prefix length is P + 1 + n and the bonus becomes the next root.      */
/* A request whose inputs do not describe such a move (n outside            */
/* [0, min(L, T - 1)], a node index outside [1, T), a negative offset or    */
/* prefix, or a tree region past total_rows) is left as it is and gets -1   */
/* for both outputs. Rows are handled whole (row_bytes = Hkv * D * esize).  */
/* ------------------------------------------------------------------------ */
void oracle_commit_kv(void *k_cache, void *v_cache, size_t row_bytes, const int64_t *kv_offsets,
                      const int32_t *prefix_lens, const int32_t *accept_len,
                      const int32_t *accepted_nodes, const int32_t *bonus, int batch, int L, int T,
                      int64_t total_rows, int32_t *new_prefix_lens, int32_t *next_roots)
{
    char *tmp = (char *)malloc(row_bytes * (size_t)(L > 0 ? L : 1) * 2);
    for (int b = 0; b < batch; ++b) {
        const int n = accept_len[b];
        const int64_t off = kv_offsets[b];
        const int64_t P = prefix_lens[b];
        const int32_t *a = accepted_nodes + (size_t)b * L;
        int ok = n >= 0 && n <= L && n <= T - 1 && off >= 0 && P >= 0 && off <= total_rows - P - T;
        for (int k = 0; ok && k < n; ++k)
            if (a[k] < 1 || a[k] >= T)
                ok = 0;
        if (!ok) {
            new_prefix_lens[b] = -1;
            if (next_roots)
                next_roots[b] = -1;
            continue;
        }
        void *caches[2] = {k_cache, v_cache};
        for (int c = 0; c < 2; ++c) {
            char *base = (char *)caches[c] + (size_t)(off + P) * row_bytes;
            for (int k = 0; k < n; ++k) /* read every source first */
                memcpy(tmp + (size_t)k * row_bytes, base + (size_t)a[k] * row_bytes, row_bytes);
            for (int k = 0; k < n; ++k)
                memcpy(base + (size_t)(1 + k) * row_bytes, tmp + (size_t)k * row_bytes, row_bytes);
        }
        new_prefix_lens[b] = (int32_t)(P + 1 + n);
        if (next_roots)
            next_roots[b] = bonus[b];
    }
    free(tmp);
}
