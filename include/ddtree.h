/*
 * ddtree.h -- C ABI of the DDTree per-round hot path on AMD Instinct MI355X
 * (gfx950): draft-tree build, tree-attention verify, greedy acceptance.
 *
 * Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
 * (Ringel, Romano), summary page, cited as [BDDT <section>].
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *    row-major and contiguous with the shapes given. The caller owns every
 *    buffer, including the workspace; the library never allocates device
 *    memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *    enqueue work and return; results are ready when the stream reaches them.
 *  - Return value: DDTREE_OK (0) or a negative DDTREE_ERR_* code. Argument
 *    checks run on the host before anything is enqueued: a call that fails
 *    them launches nothing and writes nothing. DDTREE_ERR_HIP reports a
 *    failed launch.
 *  - Workspaces hold per-call scratch only (staged top-K tables, per-split
 *    attention partials, per-node target ids); no contents carry from one
 *    call to the next, so a workspace needs no initialisation. A workspace
 *    serves one call at a time: calls that overlap on one workspace race.
 *  - dtype: DDTREE_BF16 (bfloat16 storage) or DDTREE_F32 (float32 storage).
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDTREE_VERSION 10100 /* major * 10000 + minor * 100 + patch */

typedef enum { DDTREE_BF16 = 0, DDTREE_F32 = 1 } ddtree_dtype;

enum {
    DDTREE_OK = 0,
    DDTREE_ERR_ARG = -1,         /* null pointer, size or range violation   */
    DDTREE_ERR_UNSUPPORTED = -2, /* dtype / shape outside the limits below  */
    DDTREE_ERR_WORKSPACE = -3,   /* workspace pointer missing or too small  */
    DDTREE_ERR_HIP = -4,         /* a HIP launch failed                     */
    DDTREE_ERR_SCRATCH = -5      /* ddtree_build_noalloc: the shape needs more
                                    scratch than DDTREE_BUILD_SCRATCH_MAX    */
};

/*
 * Conventions. Every call checks its arguments on the host before it
 * enqueues anything; a rejected call returns its status and has no effect.
 * A dtype argument outside the enumerators (callers may pass any int) gives
 * DDTREE_ERR_UNSUPPORTED. The *_workspace_size queries return 0 for a shape
 * outside the limits of their call; products of sizes (batch * L,
 * batch * T, batch * T * Hq) must fit in 31 bits.
 */

/* Limits. */
#define DDTREE_MAX_L 64        /* draft block length (positions)           */
#define DDTREE_MAX_K 32        /* candidates per position                  */
#define DDTREE_MAX_N 1024      /* node budget                              */
#define DDTREE_MAX_V (1 << 19) /* vocabulary                               */

/* Bits of status_flags[b] written by ddtree_build. */
#define DDTREE_STATUS_NONFINITE 1   /* a NaN or +inf logit was ranked as -inf */
#define DDTREE_STATUS_ALL_NEG_INF 2 /* a position had no finite logit         */
/* Bits of status_flags[b] written by ddtree_verify_attn. */
#define DDTREE_STATUS_OUT_NONFINITE 4 /* an output element of the request is not
                                         finite (see ddtree_verify_attn)        */
#define DDTREE_STATUS_BAD_KV 8        /* kv_offsets / prefix_lens outside the
                                         caches: the request's rows are zeros   */

/* Library version (DDTREE_VERSION of the build). Host only. */
int ddtree_version(void);

/* Static text for a return code. Host only. */
const char *ddtree_strerror(int status);

/*
 * ddtree_build -- one drafter block's per-position distributions to a
 * budget-bounded draft tree.                 [BDDT §3, §4.1, §4.2, §4.3, App. A]
 *
 * Per request b and position i (0-based, depth i+1), the row
 * logits[b, i, 0..V) is turned into log-probabilities of
 * softmax(logits / draft_temp) with a fixed, bit-reproducible arithmetic
 * (fp32 values, exact uint64 fixed-point sum, fp64 logarithm), and its K best
 * tokens (logit desc, token id asc). draft_temp = 0 is the argmax limit
 * (tied maxima share the mass, the others get -inf). NaN and +inf are ranked
 * as -inf and flagged.
 *
 * The tree is rooted at root_tokens[b] (the bonus token, node 0, depth 0,
 * score 0). N best-first pops follow: the candidate with the highest
 * cumulative log-probability (ties: shallower depth, then lower parent node
 * index, then lower rank) becomes the next node; it pushes its next sibling
 * and its best child. Scores accumulate in fp32 from the root. Nodes are
 * numbered in pop order, so parents[i] < i.
 *
 *   logits        [batch, L, V] dt                   in
 *   root_tokens   [batch] int32                      in
 *   tokens, parents, depths  [batch, N+1] int32      out (padding rows -1)
 *   scores        [batch, N+1] float32               out (padding rows -inf)
 *   num_nodes     [batch] int32                      out (root included)
 *   mask          [batch, N+1, W] uint64 or NULL     out, W = ceil((N+1)/64):
 *                 bit j of row i (word j/64, bit j%64) is set iff node j is
 *                 node i or one of its ancestors; padding rows are zero
 *   topk_tokens   [batch, L, K] int32 or NULL        out
 *   topk_logprobs [batch, L, K] float32 or NULL      out
 *   status_flags  [batch] int32 or NULL              out (DDTREE_STATUS_*)
 *   workspace     >= ddtree_build_workspace_size(...) bytes
 *
 * Limits: 1 <= batch; 1 <= L <= 64; 1 <= K <= min(32, V); 1 <= N <= 1024;
 * V <= 2^19; draft_temp >= 0 and finite.
 */
size_t ddtree_build_workspace_size(int batch, int L, int V, int K, int N);
int ddtree_build(const void *logits, ddtree_dtype dt, const int32_t *root_tokens, int batch,
                 int L, int V, int K, int N, float draft_temp, int32_t *tokens,
                 int32_t *parents, int32_t *depths, float *scores, int32_t *num_nodes,
                 uint64_t *mask, int32_t *topk_tokens, float *topk_logprobs,
                 int32_t *status_flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ddtree_build_noalloc -- ddtree_build without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, outputs, limits and return codes as ddtree_build, minus
 * the workspace. The scratch the build kernels need (per-row candidate
 * words, fixed-point sums, row maxima and flags) lives in a static device
 * array of DDTREE_BUILD_SCRATCH_MAX bytes inside the library: one copy per
 * GPU, kept until the process ends. No call allocates or frees anything.
 * A shape whose scratch, ddtree_build_workspace_size(batch, L, V, K, N),
 * exceeds DDTREE_BUILD_SCRATCH_MAX is rejected with DDTREE_ERR_SCRATCH
 * before anything is enqueued (the workloads of this library need at most
 * 0.8 MiB: e.g. 32 requests x 16 positions x V = 151936, K = 8).
 * Every call on one GPU uses that GPU's one array, whatever the stream: calls
 * that overlap on one GPU (concurrent streams or host threads) race, so
 * callers serialise them. No contents carry from one call to the next (the
 * kernels write every scratch word before reading it).
 */
#define DDTREE_BUILD_SCRATCH_MAX (4 << 20)
int ddtree_build_noalloc(const void *logits, ddtree_dtype dt, const int32_t *root_tokens,
                         int batch, int L, int V, int K, int N, float draft_temp,
                         int32_t *tokens, int32_t *parents, int32_t *depths, float *scores,
                         int32_t *num_nodes, uint64_t *mask, int32_t *topk_tokens,
                         float *topk_logprobs, int32_t *status_flags, void *stream);

/*
 * ddtree_mask -- ancestor-only attention bitmask of given trees.
 *                                                        [BDDT Abstract, §4.1]
 *   parents   [batch, T] int32 (parents[b, i] < i; -1 at the root)   in
 *   num_nodes [batch] int32 (1 <= num_nodes[b] <= T)                  in
 *   mask      [batch, T, W] uint64, W = ceil(T/64)                    out
 * Same bit layout as in ddtree_build. Limits: 1 <= T <= 1025.
 */
int ddtree_mask(const int32_t *parents, const int32_t *num_nodes, int batch, int T,
                uint64_t *mask, void *stream);

/*
 * ddtree_verify_attn -- one attention layer of the tree verification pass.
 *                                               [BDDT Abstract, §4.1, App. B]
 * Query row (b, i, h) -- node i of request b, query head h -- attends to all
 * P_b prefix keys of request b and to the tree keys j whose mask bit (i, j)
 * is set, with softmax(scale * q.k) weights over V. Query head h reads key /
 * value head h / (Hq / Hkv) (grouped-query attention).
 *
 *   q, out        [batch, T, Hq, D] dt                  in / out
 *   k, v          [rows, Hkv, D] dt                     in; request b owns rows
 *                 kv_offsets[b] .. kv_offsets[b] + P_b + T: first its P_b
 *                 prefix rows, then one row per tree node in node order
 *                 (the caller writes the tree rows before the call)
 *   kv_offsets    [batch] int64                         in
 *   prefix_lens   [batch] int32 (P_b >= 0)              in
 *   num_nodes     [batch] int32                         in; rows i >= num_nodes[b]
 *                 are written as zeros
 *   mask          [batch, T, ceil(T/64)] uint64         in (layout of ddtree_build)
 *   max_prefix_len  an upper bound on every P_b (sizes the work split)
 *   total_rows    number of rows of k and v
 *   softmax_scale <= 0 selects 1/sqrt(D)
 *   status_flags  [batch] int32 or NULL                 out: DDTREE_STATUS_OUT_NONFINITE,
 *                 DDTREE_STATUS_BAD_KV (0 when neither holds)
 *   workspace     >= ddtree_verify_workspace_size(...) bytes: the split-key
 *                 partials, and (bf16, when 16 or more 128-row tiles per
 *                 (request, kv-head) would each convert the same V tiles)
 *                 an fp16 copy of the V key tiles read, batch * Hkv *
 *                 (ceil(max_prefix_len / 64) + ceil(T / 64)) tiles of 64
 *                 keys x 128 dims; a request with P_b > max_prefix_len
 *                 converts its own tiles instead (same values)
 *
 * Request b's rows are checked on the device (the offsets and lengths may
 * come from earlier kernels): kv_offsets[b] >= 0, P_b >= 0 and
 * kv_offsets[b] + P_b + T <= total_rows. A request failing the check reads
 * no key, its output rows are zeros and it gets DDTREE_STATUS_BAD_KV; this is
 * not an error of the call.
 *
 * bf16: q.k on bf16 MFMA with fp32 accumulation; softmax in fp32; the
 * P.V product on fp16 MFMA (weights rounded to fp16, 2^-11 relative; V
 * converted to fp16, exact for |v| in [2^-14, 65280] -- the largest bf16
 * value below the fp16 limit --, smaller values rounded to fp16 subnormals).
 * A bf16 V value of magnitude 65536 or more (or a non-finite one) in the
 * key tiles of a request becomes infinite in fp16 and makes that request's
 * output rows non-finite; such a request gets DDTREE_STATUS_OUT_NONFINITE
 * (as does any output row that is not finite, e.g. from fp32 score
 * overflow). fp32 accumulation, bf16 output. f32: fp32 throughout, same
 * status bits.
 * Limits: Hq % Hkv == 0; T <= 1025; D in {32, 64, 128} (bf16: D = 128).
 */
size_t ddtree_verify_workspace_size(ddtree_dtype dt, int batch, int T, int Hq, int Hkv, int D,
                                    int max_prefix_len);
int ddtree_verify_attn(const void *q, const void *k, const void *v, ddtree_dtype dt,
                       const int64_t *kv_offsets, const int32_t *prefix_lens,
                       const int32_t *num_nodes, const uint64_t *mask, int batch, int T, int Hq,
                       int Hkv, int D, int max_prefix_len, int64_t total_rows,
                       float softmax_scale, void *out, int32_t *status_flags, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * ddtree_accept -- greedy acceptance walk.                        [BDDT §4.1]
 * The target's token after node i is argmax_v target_logits[b, i, v] (first
 * maximal index; NaN counts as -inf), or target_ids[b, i] when
 * target_logits is NULL. From the root, the walk follows the child whose
 * token equals the target's token; the matched path is accepted and the first
 * unmatched target token is the bonus (the next round's root).
 *
 *   target_logits   [batch, T, V] dt, or NULL             in
 *   target_ids      [batch, T] int32 (used when target_logits is NULL)  in
 *   tokens, parents [batch, T] int32, num_nodes [batch]   in (ddtree_build output)
 *   accepted        [batch, L] int32                      out: accepted tokens, -1 padded
 *   accepted_nodes  [batch, L] int32 or NULL              out: their node indices
 *   accept_len      [batch] int32                         out
 *   bonus           [batch] int32                         out
 *   target_argmax   [batch, T] int32 or NULL              out: the target token
 *                   per node (-1 for rows >= num_nodes[b])
 *   workspace       >= ddtree_accept_workspace_size(...) bytes: per-chunk
 *                   arg-max results (rows are split into up to 16 chunks
 *                   when batch * T is small)
 * Limits: T <= 1025, 1 <= L <= 64, V <= 2^31 - 1 (logits path: V >= 1).
 */
size_t ddtree_accept_workspace_size(int batch, int T);
int ddtree_accept(const void *target_logits, ddtree_dtype dt, const int32_t *target_ids,
                  const int32_t *tokens, const int32_t *parents, const int32_t *num_nodes,
                  int batch, int T, int V, int L, int32_t *accepted, int32_t *accepted_nodes,
                  int32_t *accept_len, int32_t *bonus, int32_t *target_argmax, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * ddtree_accept_sample -- acceptance walk at target temperature > 0.
 *                                                                [BDDT §4.1]
 * The target's token after node i of request b is a sample of
 * softmax(target_logits[b, i, :] / temperature); the walk is that of
 * ddtree_accept with these tokens in place of the arg-max. The draw is exact
 * and reproducible: with x_v = fp32(logit_v * fp32(1 / temperature)) (NaN
 * and +inf count as -inf), m = max_v x_v and the integer weights
 * u_v = rint(2^44 E(x_v - m)) of the fixed-point exponential that
 * ddtree_build uses, the token is the first v whose running sum of u exceeds
 * floor(r * S / 2^64), S = sum_v u_v, where r = word1 * 2^32 + word0 of
 * Philox4x32-10 (Salmon et al., SC 2011) with key (seed mod 2^32,
 * seed / 2^32) and counter (i, b, offset mod 2^32, offset / 2^32). A row with
 * no finite value gives token 0. Callers advance offset once per round.
 *
 *   target_logits   [batch, T, V] dt                      in
 *   tokens, parents [batch, T] int32, num_nodes [batch]   in (ddtree_build output)
 *   temperature     > 0, finite (else DDTREE_ERR_ARG)
 *   seed, offset    Philox key and the high half of its counter
 *   accepted        [batch, L] int32                      out: accepted tokens, -1 padded
 *   accepted_nodes  [batch, L] int32 or NULL              out: their node indices
 *   accept_len      [batch] int32                         out
 *   bonus           [batch] int32                         out: the sample at the last
 *                   accepted node
 *   target_tokens   [batch, T] int32 or NULL              out: the sampled token per
 *                   node (-1 for rows >= num_nodes[b])
 *   workspace       >= ddtree_accept_workspace_size(batch, T) bytes when
 *                   target_tokens is NULL (holds the sampled tokens); else
 *                   unused and may be NULL
 * Limits: T <= 1025, 1 <= L <= 64, 1 <= V <= 2^19 (the fixed-point weights
 * are below 2^45, so S stays below 2^64 exactly; DDTREE_ERR_UNSUPPORTED
 * above).
 */
int ddtree_accept_sample(const void *target_logits, ddtree_dtype dt, const int32_t *tokens,
                         const int32_t *parents, const int32_t *num_nodes, int batch, int T, int V,
                         int L, float temperature, uint64_t seed, uint64_t offset,
                         int32_t *accepted, int32_t *accepted_nodes, int32_t *accept_len,
                         int32_t *bonus, int32_t *target_tokens, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * ddtree_commit_kv -- KV compaction of the accepted path, bonus hand-off.
 *                                                                [BDDT §4.1]
 * After the verify, request b's tree K/V rows follow its prefix in node
 * order (node i at row kv_offsets[b] + prefix_lens[b] + i, as
 * ddtree_verify_attn reads them). The round commits the root (node 0, in
 * place) and the accepted nodes a_k = accepted_nodes[b, k], k < n =
 * accept_len[b]: row P + a_k moves to row P + 1 + k in both caches, every
 * move reading the rows as they were before the first (a source may be
 * another move's destination). Rows that receive no move keep their values.
 * new_prefix_lens[b] = P + 1 + n and next_roots[b] = bonus[b] (the next
 * round's root). A request whose inputs describe no such move (n outside
 * [0, min(L, T - 1)], a node index outside [1, T), a negative offset or
 * prefix, or kv_offsets[b] + P + T > total_rows) is left untouched and gets
 * -1 in both outputs; this is checked on the device and is not an error.
 *
 *   k_cache, v_cache  [total_rows, Hkv, D] dt, 16-byte aligned   in/out (in place)
 *   kv_offsets        [batch] int64, prefix_lens [batch] int32   in (as for the verify)
 *   accept_len, accepted_nodes [batch, L], bonus [batch] int32   in (ddtree_accept output)
 *   T                 tree rows per request (N + 1)
 *   new_prefix_lens   [batch] int32                              out; must not be prefix_lens
 *   next_roots        [batch] int32 or NULL                      out
 * Limits: 1 <= L <= 64, T <= 1025, D * esize a multiple of 16 and at most
 * 1024 bytes, Hkv <= 65535.
 */
int ddtree_commit_kv(void *k_cache, void *v_cache, ddtree_dtype dt, const int64_t *kv_offsets,
                     const int32_t *prefix_lens, const int32_t *accept_len,
                     const int32_t *accepted_nodes, const int32_t *bonus, int batch, int Hkv,
                     int D, int L, int T, int64_t total_rows, int32_t *new_prefix_lens,
                     int32_t *next_roots, void *stream);

/*
 * Calibration (measurement only; no part of a DDTree round calls these).
 * They give the measured peaks that roofline fractions are also reported
 * against, beside the published ones. Asynchronous on `stream`; the caller
 * times them (e.g. with events on that stream).
 *
 * ddtree_probe_mfma_bf16 -- grid workgroups of 256 threads; every wave runs
 * four independent chains of `iters` v_mfma_f32_32x32x16_bf16 operations
 * (32768 flops each), so one call performs grid * 4 * 4 * iters * 32768
 * flops with no memory traffic but the final stores.
 *   out   [grid * 256] float, device      out (sums of the accumulators)
 * Returns DDTREE_ERR_ARG for a null out or grid / iters outside [1, 2^20].
 *
 * ddtree_probe_hbm_read -- reads `bytes` from src once in 16-byte vectors
 * (grid workgroups of 256 threads, eight loads in flight per thread).
 *   src   device, 16-byte aligned, bytes a positive multiple of 16       in
 *   out   [grid] uint32, device           out (one folded word per workgroup)
 * Returns DDTREE_ERR_ARG for null pointers, misalignment or a bad size.
 */
int ddtree_probe_mfma_bf16(float *out, int grid, int iters, void *stream);
int ddtree_probe_hbm_read(const void *src, int64_t bytes, uint32_t *out, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */
