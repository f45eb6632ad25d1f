// C ABI of the DDTree hot path (declared in include/ddtree.h): argument
// validation, workspace layout and launches. Every check here runs before
// anything is enqueued, so a rejected call has no effect on the device.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/ddtree.h"
#include "ddtree_internal.h"

using namespace ddt;

// Build scratch of ddtree_build_noalloc: one copy per GPU, alive until the
// process ends. Host code never uses this name as an address (on the host it
// is a stand-in, not device memory): it takes the device address from
// hipGetSymbolAddress, per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[DDTREE_BUILD_SCRATCH_MAX];

namespace {

inline int hip_status(hipError_t e) { return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP; }

inline bool dtype_ok(int dt) { return dt == DDTREE_BF16 || dt == DDTREE_F32; }

// The dtype argument as an int. C callers (and foreign-function bindings) may
// pass any int in the enum's place; the bytes are read as an int, so a value
// outside the enumerators is rejected rather than loaded as an enum.
inline int dtype_value(const ddtree_dtype* d) {
  int v;
  static_assert(sizeof(v) == sizeof(*d), "enum and int differ in size");
  memcpy(&v, d, sizeof v);
  return v;
}

// a * b * c <= 2^31 - 1 for positive a, b, c, decided without forming a
// product that could overflow
inline bool product_fits_i32(long long a, long long b, long long c = 1) {
  const long long lim = 0x7FFFFFFFLL;
  return a <= lim / b && a * b <= lim / c;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DDTREE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DDTREE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DDTREE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DDTREE_OK;
}

}  // namespace

extern "C" {

int ddtree_version(void) { return DDTREE_VERSION; }

const char* ddtree_strerror(int status) {
  switch (status) {
    case DDTREE_OK: return "ok";
    case DDTREE_ERR_ARG: return "invalid argument (null pointer, size or range)";
    case DDTREE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case DDTREE_ERR_WORKSPACE: return "workspace missing or too small";
    case DDTREE_ERR_HIP: return "HIP launch failed";
    case DDTREE_ERR_SCRATCH:
      return "shape needs more build scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

size_t ddtree_build_workspace_size(int batch, int L, int V, int K, int N) {
  (void)N;
  if (batch < 1 || L < 1 || K < 1 || V < 1) return 0;
  if (L > DDTREE_MAX_L || K > DDTREE_MAX_K || V > DDTREE_MAX_V) return 0;
  if (!product_fits_i32(batch, L)) return 0;
  return build_workspace_bytes(batch, L, V, K);
}

}  // extern "C"

namespace {

// Argument checks of ddtree_build other than the workspace (host only).
int build_check(const void* logits, int dt, const int32_t* root_tokens, int batch, int L, int V,
                int K, int N, float draft_temp, const int32_t* tokens, const int32_t* parents,
                const int32_t* depths, const float* scores, const int32_t* num_nodes) {
  if (!logits || !root_tokens || !tokens || !parents || !depths || !scores || !num_nodes)
    return DDTREE_ERR_ARG;
  if (batch < 1 || L < 1 || V < 1 || K < 1 || N < 1) return DDTREE_ERR_ARG;
  if (K > V) return DDTREE_ERR_ARG;
  if (!(draft_temp >= 0.0f) || isinf(draft_temp)) return DDTREE_ERR_ARG;
  if (!dtype_ok(dt)) return DDTREE_ERR_UNSUPPORTED;
  if (L > DDTREE_MAX_L || K > DDTREE_MAX_K || N > DDTREE_MAX_N || V > DDTREE_MAX_V)
    return DDTREE_ERR_UNSUPPORTED;
  if (!product_fits_i32(batch, L)) return DDTREE_ERR_UNSUPPORTED;
  return DDTREE_OK;
}

int build_launch(const void* logits, int dt, const int32_t* root_tokens, int batch, int L, int V,
                 int K, int N, float draft_temp, int32_t* tokens, int32_t* parents,
                 int32_t* depths, float* scores, int32_t* num_nodes, uint64_t* mask,
                 int32_t* topk_tokens, float* topk_logprobs, int32_t* status_flags,
                 void* workspace, size_t workspace_bytes, void* stream) {
  BuildArgs a{};
  a.logits = logits;
  a.dtype = dt;
  a.root_tokens = root_tokens;
  a.batch = batch;
  a.L = L;
  a.V = V;
  a.K = K;
  a.N = N;
  if (draft_temp == 0.0f) {
    a.mode = 2;
    a.inv_tau = 1.0f;
  } else {
    a.inv_tau = 1.0f / draft_temp;
    a.mode = (a.inv_tau == 1.0f) ? 0 : 1;
  }
  a.tokens = tokens;
  a.parents = parents;
  a.depths = depths;
  a.scores = scores;
  a.num_nodes = num_nodes;
  a.mask = mask;
  a.status = status_flags;
  a.topk_tok = topk_tokens;
  a.topk_lp = topk_logprobs;
  return hip_status(launch_build(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int ddtree_build(const void* logits, ddtree_dtype dt_arg, const int32_t* root_tokens, int batch,
                 int L, int V, int K, int N, float draft_temp, int32_t* tokens,
                 int32_t* parents, int32_t* depths, float* scores, int32_t* num_nodes,
                 uint64_t* mask, int32_t* topk_tokens, float* topk_logprobs,
                 int32_t* status_flags, void* workspace, size_t workspace_bytes, void* stream) {
  const int dt = dtype_value(&dt_arg);
  const int chk = build_check(logits, dt, root_tokens, batch, L, V, K, N, draft_temp, tokens,
                              parents, depths, scores, num_nodes);
  if (chk != DDTREE_OK) return chk;
  const size_t need = build_workspace_bytes(batch, L, V, K);
  if (!workspace || workspace_bytes < need) return DDTREE_ERR_WORKSPACE;
  return build_launch(logits, dt, root_tokens, batch, L, V, K, N, draft_temp, tokens, parents,
                      depths, scores, num_nodes, mask, topk_tokens, topk_logprobs, status_flags,
                      workspace, workspace_bytes, stream);
}

int ddtree_build_noalloc(const void* logits, ddtree_dtype dt_arg, const int32_t* root_tokens,
                         int batch, int L, int V, int K, int N, float draft_temp,
                         int32_t* tokens, int32_t* parents, int32_t* depths, float* scores,
                         int32_t* num_nodes, uint64_t* mask, int32_t* topk_tokens,
                         float* topk_logprobs, int32_t* status_flags, void* stream) {
  const int dt = dtype_value(&dt_arg);
  const int chk = build_check(logits, dt, root_tokens, batch, L, V, K, N, draft_temp, tokens,
                              parents, depths, scores, num_nodes);
  if (chk != DDTREE_OK) return chk;
  if (build_workspace_bytes(batch, L, V, K) > (size_t)DDTREE_BUILD_SCRATCH_MAX)
    return DDTREE_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != DDTREE_OK) return st;
  return build_launch(logits, dt, root_tokens, batch, L, V, K, N, draft_temp, tokens, parents,
                      depths, scores, num_nodes, mask, topk_tokens, topk_logprobs, status_flags,
                      ws, (size_t)DDTREE_BUILD_SCRATCH_MAX, stream);
}

int ddtree_mask(const int32_t* parents, const int32_t* num_nodes, int batch, int T,
                uint64_t* mask, void* stream) {
  if (!parents || !num_nodes || !mask) return DDTREE_ERR_ARG;
  if (batch < 1 || T < 1) return DDTREE_ERR_ARG;
  if (T > DDTREE_MAX_N + 1) return DDTREE_ERR_UNSUPPORTED;
  return hip_status(launch_mask(parents, num_nodes, batch, T, mask,
                                static_cast<hipStream_t>(stream)));
}

size_t ddtree_verify_workspace_size(ddtree_dtype dt_arg, int batch, int T, int Hq, int Hkv, int D,
                                    int max_prefix_len) {
  const int dt = dtype_value(&dt_arg);
  if (batch < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_prefix_len < 0) return 0;
  if (Hq % Hkv != 0 || !dtype_ok(dt) || T > DDTREE_MAX_N + 1) return 0;
  if (D != 32 && D != 64 && D != 128) return 0;
  if (dt == DDTREE_BF16 && D != 128) return 0;
  if (!product_fits_i32(batch, T, Hq)) return 0;
  return attn_workspace_bytes(dt, batch, T, Hq, Hkv, D, max_prefix_len);
}

int ddtree_verify_attn(const void* q, const void* k, const void* v, ddtree_dtype dt_arg,
                       const int64_t* kv_offsets, const int32_t* prefix_lens,
                       const int32_t* num_nodes, const uint64_t* mask, int batch, int T, int Hq,
                       int Hkv, int D, int max_prefix_len, int64_t total_rows,
                       float softmax_scale, void* out, int32_t* status_flags, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const int dt = dtype_value(&dt_arg);
  if (!q || !k || !v || !kv_offsets || !prefix_lens || !num_nodes || !mask || !out)
    return DDTREE_ERR_ARG;
  if (batch < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_prefix_len < 0 || total_rows < 1)
    return DDTREE_ERR_ARG;
  if (Hq % Hkv != 0) return DDTREE_ERR_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return DDTREE_ERR_ARG;
  if (!dtype_ok(dt)) return DDTREE_ERR_UNSUPPORTED;
  if (T > DDTREE_MAX_N + 1) return DDTREE_ERR_UNSUPPORTED;
  if (D != 32 && D != 64 && D != 128) return DDTREE_ERR_UNSUPPORTED;
  if (dt == DDTREE_BF16 && D != 128) return DDTREE_ERR_UNSUPPORTED;
  if (!product_fits_i32(batch, T, Hq)) return DDTREE_ERR_UNSUPPORTED;
  const size_t need = attn_workspace_bytes(dt, batch, T, Hq, Hkv, D, max_prefix_len);
  if (need == 0) return DDTREE_ERR_UNSUPPORTED;  // the work grid would not fit a launch
  if (!workspace || workspace_bytes < need) return DDTREE_ERR_WORKSPACE;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dtype = dt;
  a.kv_offsets = kv_offsets;
  a.prefix_lens = prefix_lens;
  a.num_nodes = num_nodes;
  a.mask = mask;
  a.batch = batch;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.max_prefix_len = max_prefix_len;
  a.total_rows = total_rows;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)D);
  a.out = out;
  a.status = status_flags;
  return hip_status(launch_attn(a, workspace, static_cast<hipStream_t>(stream)));
}

size_t ddtree_accept_workspace_size(int batch, int T) {
  if (batch < 1 || T < 1 || T > DDTREE_MAX_N + 1) return 0;
  if (!product_fits_i32(batch, T)) return 0;
  return accept_workspace_bytes(batch, T);
}

int ddtree_accept(const void* target_logits, ddtree_dtype dt_arg, const int32_t* target_ids,
                  const int32_t* tokens, const int32_t* parents, const int32_t* num_nodes,
                  int batch, int T, int V, int L, int32_t* accepted, int32_t* accepted_nodes,
                  int32_t* accept_len, int32_t* bonus, int32_t* target_argmax, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const int dt = dtype_value(&dt_arg);
  if (!tokens || !parents || !num_nodes || !accepted || !accept_len || !bonus)
    return DDTREE_ERR_ARG;
  if (!target_logits && !target_ids) return DDTREE_ERR_ARG;
  if (batch < 1 || T < 1 || L < 1) return DDTREE_ERR_ARG;
  if (target_logits && V < 1) return DDTREE_ERR_ARG;
  if (target_logits && !dtype_ok(dt)) return DDTREE_ERR_UNSUPPORTED;
  if (T > DDTREE_MAX_N + 1 || L > DDTREE_MAX_L) return DDTREE_ERR_UNSUPPORTED;
  if (!product_fits_i32(batch, T)) return DDTREE_ERR_UNSUPPORTED;
  const size_t need = accept_workspace_bytes(batch, T);
  if (!workspace || workspace_bytes < need) return DDTREE_ERR_WORKSPACE;
  AcceptArgs a{};
  a.target_logits = target_logits;
  a.dtype = dt;
  a.target_ids = target_ids;
  a.tokens = tokens;
  a.parents = parents;
  a.num_nodes = num_nodes;
  a.batch = batch;
  a.T = T;
  a.V = V;
  a.L = L;
  a.accepted = accepted;
  a.accepted_nodes = accepted_nodes;
  a.accept_len = accept_len;
  a.bonus = bonus;
  a.target_argmax = target_argmax;
  const AcceptWork w = accept_carve(workspace, batch, T);
  return hip_status(launch_accept(a, w, static_cast<hipStream_t>(stream)));
}

int ddtree_accept_sample(const void* target_logits, ddtree_dtype dt_arg, const int32_t* tokens,
                         const int32_t* parents, const int32_t* num_nodes, int batch, int T, int V,
                         int L, float temperature, uint64_t seed, uint64_t offset,
                         int32_t* accepted, int32_t* accepted_nodes, int32_t* accept_len,
                         int32_t* bonus, int32_t* target_tokens, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int dt = dtype_value(&dt_arg);
  if (!target_logits || !tokens || !parents || !num_nodes || !accepted || !accept_len || !bonus)
    return DDTREE_ERR_ARG;
  if (batch < 1 || T < 1 || L < 1 || V < 1) return DDTREE_ERR_ARG;
  if (!(temperature > 0.0f) || isinf(temperature)) return DDTREE_ERR_ARG;
  if (!dtype_ok(dt)) return DDTREE_ERR_UNSUPPORTED;
  if (T > DDTREE_MAX_N + 1 || L > DDTREE_MAX_L) return DDTREE_ERR_UNSUPPORTED;
  // each weight is below 2^45: V <= 2^19 keeps the 64-bit row sum exact
  if (V > DDTREE_MAX_V) return DDTREE_ERR_UNSUPPORTED;
  if (!product_fits_i32(batch, T)) return DDTREE_ERR_UNSUPPORTED;
  if (!target_tokens && (!workspace || workspace_bytes < accept_workspace_bytes(batch, T)))
    return DDTREE_ERR_WORKSPACE;
  AcceptArgs a{};
  a.target_logits = target_logits;
  a.dtype = dt;
  a.tokens = tokens;
  a.parents = parents;
  a.num_nodes = num_nodes;
  a.batch = batch;
  a.T = T;
  a.V = V;
  a.L = L;
  a.accepted = accepted;
  a.accepted_nodes = accepted_nodes;
  a.accept_len = accept_len;
  a.bonus = bonus;
  int32_t* tgt = target_tokens ? target_tokens : static_cast<int32_t*>(workspace);
  const float inv_tau = 1.0f / temperature;
  return hip_status(launch_accept_sample(a, inv_tau, seed, offset, tgt,
                                         static_cast<hipStream_t>(stream)));
}

int ddtree_commit_kv(void* k_cache, void* v_cache, ddtree_dtype dt_arg, const int64_t* kv_offsets,
                     const int32_t* prefix_lens, const int32_t* accept_len,
                     const int32_t* accepted_nodes, const int32_t* bonus, int batch, int Hkv,
                     int D, int L, int T, int64_t total_rows, int32_t* new_prefix_lens,
                     int32_t* next_roots, void* stream) {
  const int dt = dtype_value(&dt_arg);
  if (!k_cache || !v_cache || !kv_offsets || !prefix_lens || !accept_len || !accepted_nodes ||
      !bonus || !new_prefix_lens)
    return DDTREE_ERR_ARG;
  if (batch < 1 || Hkv < 1 || D < 1 || L < 1 || T < 1 || total_rows < 1) return DDTREE_ERR_ARG;
  if (new_prefix_lens == prefix_lens) return DDTREE_ERR_ARG;
  if (!dtype_ok(dt)) return DDTREE_ERR_UNSUPPORTED;
  if (L > DDTREE_MAX_L || T > DDTREE_MAX_N + 1 || Hkv > 65535) return DDTREE_ERR_UNSUPPORTED;
  const long long slice = (long long)D * (dt == DDTREE_BF16 ? 2 : 4);
  if (slice % 16 != 0 || slice > 1024) return DDTREE_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(k_cache) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(v_cache) % 16 != 0)
    return DDTREE_ERR_UNSUPPORTED;
  CommitArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_offsets = kv_offsets;
  a.prefix_lens = prefix_lens;
  a.accept_len = accept_len;
  a.accepted_nodes = accepted_nodes;
  a.bonus = bonus;
  a.batch = batch;
  a.Hkv = Hkv;
  a.L = L;
  a.T = T;
  a.cpr = (int)(slice / 16);
  a.total_rows = total_rows;
  a.new_prefix_lens = new_prefix_lens;
  a.next_roots = next_roots;
  return hip_status(launch_commit(a, static_cast<hipStream_t>(stream)));
}

int ddtree_probe_mfma_bf16(float* out, int grid, int iters, void* stream) {
  if (!out || grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 20)) return DDTREE_ERR_ARG;
  return hip_status(launch_probe_mfma(out, grid, iters, static_cast<hipStream_t>(stream)));
}

int ddtree_probe_hbm_read(const void* src, int64_t bytes, uint32_t* out, int grid, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > (1 << 20))
    return DDTREE_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return DDTREE_ERR_ARG;
  return hip_status(launch_probe_read(src, bytes, out, grid, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
