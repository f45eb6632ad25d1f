// Greedy acceptance on gfx950: target argmax per tree node, then the walk.
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, §4.1: the tree is walked with the target's
// decoding rule; the matched path is accepted and the first unmatched target
// token becomes the next bonus token. At temperature 0 the rule is argmax.
//
// k_argmax: one workgroup per (request, node) row of the target logits,
// streamed once with 16-byte loads (8 in flight per thread); rows past
// num_nodes are skipped. k_walk: one wavefront per request, at most L steps,
// each a ballot over the current node's children.
#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

constexpr int kMaxT = 1025;

// (value desc, index asc): is (v2, i2) better than (v1, i1)?
__device__ __forceinline__ bool better(float v2, int i2, float v1, int i1) {
  return v2 > v1 || (v2 == v1 && i2 < i1);
}

__device__ void walk_wave(const AcceptArgs& a, int b, const int32_t* tgt_row, int32_t* s_tok,
                          int32_t* s_par, int32_t* s_tgt) {
  const int lane = threadIdx.x & 63;
  const int T = a.T;
  const int nn = min(a.num_nodes[b], T);
  for (int i = lane; i < T; i += 64) {
    s_tok[i] = a.tokens[(size_t)b * T + i];
    s_par[i] = a.parents[(size_t)b * T + i];
    s_tgt[i] = tgt_row[i];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  int cur = 0, len = 0, bonus = -1;
  for (;;) {
    const int y = s_tgt[cur];
    int next = -1;
    for (int c0 = cur + 1; c0 < nn; c0 += 64) {
      const int c = c0 + lane;
      const bool hit = c < nn && s_par[c] == cur && s_tok[c] == y;
      const uint64_t bal = __ballot(hit);
      if (bal) {
        next = c0 + __builtin_ctzll(bal);
        break;
      }
    }
    if (next < 0 || len >= a.L) {
      bonus = y;
      break;
    }
    if (lane == 0) {
      a.accepted[(size_t)b * a.L + len] = y;
      if (a.accepted_nodes) a.accepted_nodes[(size_t)b * a.L + len] = next;
    }
    ++len;
    cur = next;
  }
  for (int k = len + lane; k < a.L; k += 64) {
    a.accepted[(size_t)b * a.L + k] = -1;
    if (a.accepted_nodes) a.accepted_nodes[(size_t)b * a.L + k] = -1;
  }
  if (lane == 0) {
    a.accept_len[b] = len;
    a.bonus[b] = bonus;
  }
}

template <typename IN_T, int BLOCK, bool VEC>
__global__ __launch_bounds__(BLOCK) void k_argmax(AcceptArgs a) {
  __shared__ float s_v[BLOCK / 64];
  __shared__ int s_i[BLOCK / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T;
  const int rowi = blockIdx.x;
  const int b = rowi / T, i = rowi - (rowi / T) * T;
  const int nn = min(a.num_nodes[b], T);
  int32_t* tgt = a.target_argmax;

  if (i < nn) {
    const IN_T* row = static_cast<const IN_T*>(a.target_logits) + (size_t)rowi * a.V;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    if constexpr (VEC) {
      constexpr int EPV = 16 / sizeof(IN_T);
      constexpr int U = 8;  // 16-byte loads in flight per thread
      const int nvec = a.V / EPV;
      const uint4* p = reinterpret_cast<const uint4*>(row);
      if (tid < nvec) bi = tid * EPV;
      for (int base = tid; base < nvec; base += BLOCK * U) {
        uint4 u[U];
#pragma unroll
        for (int j = 0; j < U; ++j) u[j] = p[min(base + j * BLOCK, nvec - 1)];  // clamped: always in bounds
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const int vi = base + j * BLOCK;
          if (vi >= nvec) break;
          const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
          if constexpr (sizeof(IN_T) == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x0 = __uint_as_float(w[q] << 16);
              const float x1 = __uint_as_float(w[q] & 0xFFFF0000u);
              if (x0 > best) { best = x0; bi = vi * EPV + 2 * q; }
              if (x1 > best) { best = x1; bi = vi * EPV + 2 * q + 1; }
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x = __uint_as_float(w[q]);
              if (x > best) { best = x; bi = vi * EPV + q; }
            }
          }
        }
      }
    } else {
      if (tid < a.V) bi = tid;
      for (int v = tid; v < a.V; v += BLOCK) {
        float x;
        if constexpr (sizeof(IN_T) == 2) x = bf16_to_float(reinterpret_cast<const uint16_t*>(row)[v]);
        else x = reinterpret_cast<const float*>(row)[v];
        if (x > best) { best = x; bi = v; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
    }
    if (lane == 0) { s_v[wid] = best; s_i[wid] = bi; }
    __syncthreads();
    if (tid == 0) {
      float bv = s_v[0];
      int bx = s_i[0];
      for (int w2 = 1; w2 < BLOCK / 64; ++w2)
        if (better(s_v[w2], s_i[w2], bv, bx)) { bv = s_v[w2]; bx = s_i[w2]; }
      tgt[rowi] = bx;
    }
  } else if (tid == 0) {
    tgt[rowi] = -1;
  }

}

// Walk only, from given target ids.
__global__ __launch_bounds__(64) void k_walk_ids(AcceptArgs a) {
  __shared__ int32_t s_tok[kMaxT], s_par[kMaxT], s_tgt[kMaxT];
  const int b = blockIdx.x;
  const int nn = min(a.num_nodes[b], a.T);
  if (a.target_argmax) {
    for (int i = threadIdx.x; i < a.T; i += 64)
      a.target_argmax[(size_t)b * a.T + i] = i < nn ? a.target_ids[(size_t)b * a.T + i] : -1;
  }
  walk_wave(a, b, a.target_ids + (size_t)b * a.T, s_tok, s_par, s_tgt);
}

// The walk of one request from its per-node target tokens.
__global__ __launch_bounds__(64) void k_walk(AcceptArgs a) {
  __shared__ int32_t s_tok[kMaxT], s_par[kMaxT], s_tgt[kMaxT];
  const int b = blockIdx.x;
  walk_wave(a, b, a.target_argmax + (size_t)b * a.T, s_tok, s_par, s_tgt);
}

template <typename IN_T>
hipError_t launch_logits(const AcceptArgs& a, hipStream_t st) {
  const bool vec = (reinterpret_cast<uintptr_t>(a.target_logits) % 16 == 0) &&
                   ((size_t)a.V * sizeof(IN_T)) % 16 == 0;
  dim3 grid(a.batch * a.T);
  if (vec)
    hipLaunchKernelGGL((k_argmax<IN_T, 256, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_argmax<IN_T, 256, false>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_walk, dim3(a.batch), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t accept_workspace_bytes(int batch, int T) { return align_up((size_t)batch * T * 4, 256); }

void accept_carve(void* ws, int batch, int T, int32_t** tgt) {
  (void)batch;
  (void)T;
  *tgt = reinterpret_cast<int32_t*>(ws);
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t st) {
  if (!a.target_logits) {
    hipLaunchKernelGGL(k_walk_ids, dim3(a.batch), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  if (a.dtype == 0) return launch_logits<uint16_t>(a, st);
  return launch_logits<float>(a, st);
}

}  // namespace ddt
