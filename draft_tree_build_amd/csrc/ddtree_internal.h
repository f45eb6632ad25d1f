// Host-side launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ddt {

// ---------------------------------------------------------------- build
struct BuildArgs {
  const void* logits;       // [batch, L, V]
  int dtype;                // 0 bf16, 1 f32
  const int32_t* root_tokens;
  int batch, L, V, K, N;
  int mode;                 // 0: tau == 1, 1: tau > 0 (scale by inv_tau), 2: tau == 0 (argmax)
  float inv_tau;
  int32_t* tokens;
  int32_t* parents;
  int32_t* depths;
  float* scores;
  int32_t* num_nodes;
  uint64_t* mask;           // may be null
  int32_t* topk_tok;        // [batch, L, K] or null
  float* topk_lp;           // [batch, L, K] or null
  int32_t* status;          // may be null
  // workspace: per-row results of the row stage
  uint64_t* row_cand;       // [rows, K] candidate words, best first
  uint64_t* row_sum;        // [rows, S] fixed-point partial sums
  float* row_max;           // [rows]
  int32_t* row_flags;       // [rows]
  // workspace: per-chunk results of split rows (S > 1)
  uint64_t* part_cand;      // [rows, S, K]
  float* part_max;          // [rows, S]
  int32_t* part_flags;      // [rows, S]
};
struct RowPlan {
  int S;        // chunks per row (1: no split)
  int cv;       // 16-byte vectors per chunk
  bool vec_ok;  // rows are 16-byte aligned
};
RowPlan plan_rows(int batch, int L, int V, int K, int esize, bool vec_ok);
size_t build_workspace_bytes(int batch, int L, int V, int K);
// Workspace layout for S chunks per row; fills the workspace pointers of `a`
// when ws and a are given. Returns the bytes needed.
size_t build_layout(int batch, int L, int K, int S, void* ws, BuildArgs* a);
hipError_t launch_build(BuildArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

struct TreeArgs {
  const uint64_t* row_cand; // [batch * L, K]
  const uint64_t* row_sum;  // [batch * L, S]
  const float* row_max;
  const int32_t* row_flags;
  int S;
  int mode;
  const int32_t* root_tokens;
  int L, K, N;
  int32_t* tokens;
  int32_t* parents;
  int32_t* depths;
  float* scores;
  int32_t* num_nodes;
  uint64_t* mask;           // may be null
  int32_t* topk_tok;        // may be null
  float* topk_lp;           // may be null
  int32_t* status;          // may be null
};
hipError_t launch_tree(const TreeArgs& t, int batch, hipStream_t stream);

hipError_t launch_mask(const int32_t* parents, const int32_t* num_nodes, int batch, int T,
                       uint64_t* mask, hipStream_t stream);

// ---------------------------------------------------------------- verify
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int dtype;
  const int64_t* kv_offsets;
  const int32_t* prefix_lens;
  const int32_t* num_nodes;
  const uint64_t* mask;
  int batch, T, Hq, Hkv, D;
  int max_prefix_len;
  int64_t total_rows;
  float scale;
  void* out;
  int32_t* status;          // [batch] or null: DDTREE_STATUS_OUT_NONFINITE / _BAD_KV
};
size_t attn_workspace_bytes(int dtype, int batch, int T, int Hq, int Hkv, int D,
                            int max_prefix_len);
hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- accept
struct AcceptArgs {
  const void* target_logits;  // may be null
  int dtype;
  const int32_t* target_ids;  // used when target_logits is null
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* num_nodes;
  int batch, T, V, L;
  int32_t* accepted;
  int32_t* accepted_nodes;    // may be null
  int32_t* accept_len;
  int32_t* bonus;
  int32_t* target_argmax;     // may be null
};
// Per-chunk arg-max results in the accept workspace: S2 chunks per row.
struct AcceptWork {
  int S2;
  float* pv;
  int32_t* pidx;
};
int accept_splits(int batch, int T);
size_t accept_workspace_bytes(int batch, int T);
AcceptWork accept_carve(void* ws, int batch, int T);
hipError_t launch_accept(const AcceptArgs& a, const AcceptWork& w, hipStream_t stream);
// tgt: [batch, T] sampled tokens (-1 past num_nodes), then the walk from them
hipError_t launch_accept_sample(const AcceptArgs& a, float inv_tau, uint64_t seed, uint64_t offset,
                                int32_t* tgt, hipStream_t stream);

// ---------------------------------------------------------------- commit
struct CommitArgs {
  void* k_cache;
  void* v_cache;
  const int64_t* kv_offsets;
  const int32_t* prefix_lens;
  const int32_t* accept_len;
  const int32_t* accepted_nodes;  // [batch, L]
  const int32_t* bonus;
  int batch, Hkv, L, T;
  int cpr;                        // 16-byte chunks per head slice of a row (D * esize / 16)
  int64_t total_rows;
  int32_t* new_prefix_lens;
  int32_t* next_roots;            // may be null
};
hipError_t launch_commit(const CommitArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- calibration
hipError_t launch_probe_mfma(float* out, int grid, int iters, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int grid,
                             hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace ddt
