// Greedy acceptance on gfx950: target argmax per tree node, then the walk.
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, §4.1: the tree is walked with the target's
// decoding rule; the matched path is accepted and the first unmatched target
// token becomes the next bonus token. At temperature 0 the rule is argmax.
//
// k_argmax: one workgroup per chunk of a (request, node) row of the target
// logits (S2 chunks per row, so that small batches still fill the chip),
// streamed once with 16-byte loads; rows past num_nodes are skipped. It
// leaves the chunk's (maximum, first index) in the workspace. k_walk: one
// workgroup per request: it reduces the chunk results to the target token of
// every node, finds for every node its first child carrying that token (all
// nodes at once), then follows that pointer from the root for at most L
// steps.
#include <algorithm>

#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

constexpr int kMaxT = 1025;
constexpr int kNoChild = 0x7FFFFFFF;

// (value desc, index asc): is (v2, i2) better than (v1, i1)?
__device__ __forceinline__ bool better(float v2, int i2, float v1, int i1) {
  return v2 > v1 || (v2 == v1 && i2 < i1);
}

// One step of the wave arg-max: the pair CTRL brings in, where better.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = __uint_as_float(dpp_src<CTRL, ROW_MASK>(__float_as_uint(-INFINITY), __float_as_uint(v)));
  const int oi = (int)dpp_src<CTRL, ROW_MASK>((uint32_t)kNoChild, (uint32_t)i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}
// Arg-max over the 64 lanes (DPP steps as in dpp_reduce), returned uniform.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0xB1, 0xF>(v, i);
  argmax_step<0x4E, 0xF>(v, i);
  argmax_step<0x141, 0xF>(v, i);
  argmax_step<0x140, 0xF>(v, i);
  argmax_step<0x142, 0xA>(v, i);
  argmax_step<0x143, 0xC>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// Chunk s of row (b, i): blockIdx.x = row * S2 + s. Writes the chunk's
// maximum and first maximal index (NaN counts as -inf; a chunk of only
// -inf / NaN reports its first index, an empty chunk index kNoChild).
template <typename IN_T, int BLOCK, bool VEC, int U>
__global__ __launch_bounds__(BLOCK) void k_argmax(AcceptArgs a, int S2, float* pv, int32_t* pidx) {
  constexpr int NW = BLOCK / 64;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T;
  const int rowi = (int)blockIdx.x / S2, s = (int)blockIdx.x - rowi * S2;
  const int b = rowi / T, i = rowi - b * T;
  if (i >= min(a.num_nodes[b], T)) return;  // no node: the walk never reads it
  const IN_T* row = static_cast<const IN_T*>(a.target_logits) + (size_t)rowi * a.V;
  float best = -INFINITY;
  int bi = kNoChild;
  if constexpr (VEC) {
    constexpr int EPV = 16 / sizeof(IN_T);  // U: 16-byte loads in flight per thread
    const int nvec = a.V / EPV;
    const int cv = (nvec + S2 - 1) / S2;
    const int v0 = s * cv, v1 = min(v0 + cv, nvec);
    const uint4* p = reinterpret_cast<const uint4*>(row);
    if (v0 + tid < v1) bi = (v0 + tid) * EPV;
    for (int base = v0 + tid; base < v1; base += BLOCK * U) {
      uint4 u[U];
#pragma unroll
      for (int j = 0; j < U; ++j) u[j] = p[min(base + j * BLOCK, v1 - 1)];  // clamped: always in bounds
      // all U loads are issued before the first use (keeps the compiler
      // from sinking each load into the guarded block that consumes it)
#pragma unroll
      for (int j = 0; j < U; ++j) asm volatile("" : "+v"(u[j].x), "+v"(u[j].y), "+v"(u[j].z), "+v"(u[j].w));
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int vi = base + j * BLOCK;
        if (vi >= v1) break;
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
    const int ce = (a.V + S2 - 1) / S2;
    const int e0 = s * ce, e1 = min(e0 + ce, a.V);
    if (e0 + tid < e1) bi = e0 + tid;
    for (int v = e0 + tid; v < e1; v += BLOCK) {
      float x;
      if constexpr (sizeof(IN_T) == 2) x = bf16_to_float(reinterpret_cast<const uint16_t*>(row)[v]);
      else x = reinterpret_cast<const float*>(row)[v];
      if (x > best) { best = x; bi = v; }
    }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    s_v[wid] = best;
    s_i[wid] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = s_v[0];
    int bx = s_i[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2)
      if (better(s_v[w2], s_i[w2], bv, bx)) { bv = s_v[w2]; bx = s_i[w2]; }
    pv[blockIdx.x] = bv;
    pidx[blockIdx.x] = bx;
  }
}

// One workgroup per request (BLOCK >= T where possible: each node's inputs
// are fetched in one round trip). IDS: target tokens from target_ids; else
// from the S2 chunk results per row of k_argmax.
template <bool IDS, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_walk(AcceptArgs a, int S2, const float* pv,
                                                const int32_t* pidx) {
  __shared__ int32_t s_tok[kMaxT], s_par[kMaxT], s_tgt[kMaxT], s_next[kMaxT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x;
  const int T = a.T;
  const int nn = min(a.num_nodes[b], T);
  const size_t r0 = (size_t)b * T;
  for (int i = tid; i < T; i += BLOCK) {
    const int32_t tk = a.tokens[r0 + i], pa = a.parents[r0 + i];
    int y = -1;
    if (i < nn) {
      if constexpr (!IDS) {
        // all S2 <= 16 chunk results are requested before the first compare
        const size_t q = (r0 + i) * S2;
        float cv[16];
        int ci[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          cv[s] = s < S2 ? pv[q + s] : -INFINITY;
          ci[s] = s < S2 ? pidx[q + s] : kNoChild;
        }
        float bv = cv[0];
        int bx = ci[0];
#pragma unroll
        for (int s = 1; s < 16; ++s)
          if (better(cv[s], ci[s], bv, bx)) { bv = cv[s]; bx = ci[s]; }
        y = bx;
      } else {
        y = a.target_ids[r0 + i];
      }
    }
    if (a.target_argmax) a.target_argmax[r0 + i] = y;
    s_tgt[i] = y;
    s_tok[i] = tk;
    s_par[i] = pa;
    s_next[i] = kNoChild;
  }
  __syncthreads();
  // the first child (lowest index) of every node whose token is the node's
  // target token; a parent index not below the child's (malformed) is skipped
  for (int c = 1 + tid; c < nn; c += BLOCK) {
    const int p = s_par[c];
    if (p >= 0 && p < c && s_tok[c] == s_tgt[p]) atomicMin(&s_next[p], c);
  }
  __syncthreads();
  if (tid >= 64) return;
  int32_t* acc = a.accepted + (size_t)b * a.L;
  int32_t* accn = a.accepted_nodes ? a.accepted_nodes + (size_t)b * a.L : nullptr;
  int cur = 0, len = 0, bonus;
  if (T <= 128) {
    // small trees: next and target of node j sit in lane j % 64 of two
    // registers, so each step is a pair of lane reads (no LDS round trip)
    const int n0 = s_next[lane], t0 = s_tgt[lane];
    const int n1 = lane + 64 < T ? s_next[lane + 64] : kNoChild;
    const int t1 = lane + 64 < T ? s_tgt[lane + 64] : -1;
    for (;;) {
      const int nx = cur < 64 ? __builtin_amdgcn_readlane(n0, cur) : __builtin_amdgcn_readlane(n1, cur - 64);
      const int y = cur < 64 ? __builtin_amdgcn_readlane(t0, cur) : __builtin_amdgcn_readlane(t1, cur - 64);
      if (nx == kNoChild || len >= a.L) {
        bonus = y;
        break;
      }
      if (lane == 0) {
        acc[len] = y;
        if (accn) accn[len] = nx;
      }
      ++len;
      cur = nx;
    }
  } else {
    for (;;) {
      const int nx = s_next[cur], y = s_tgt[cur];
      if (nx == kNoChild || len >= a.L) {
        bonus = y;
        break;
      }
      if (lane == 0) {
        acc[len] = y;
        if (accn) accn[len] = nx;
      }
      ++len;
      cur = nx;
    }
  }
  for (int k = len + lane; k < a.L; k += 64) {
    acc[k] = -1;
    if (accn) accn[k] = -1;
  }
  if (lane == 0) {
    a.accept_len[b] = len;
    a.bonus[b] = bonus;
  }
}

// ---------------------------------------------------------------------------
// Acceptance at target temperature tau > 0 [BDDT §4.1]: the target's token
// after node i is a sample of softmax(logits_i / tau). The weights are the
// fixed-point terms of the numerics spec, u_v = rint(2^44 E(x_v - m)) with
// x_v = fp32(logit_v * inv_tau) (NaN, +inf -> -inf) and m = max_v x_v; the
// uniform r (64 bits) is Philox4x32-10 (Salmon et al., SC 2011) with key
// (seed_lo, seed_hi) and counter (i, b, offset_lo, offset_hi), r = word1 *
// 2^32 + word0; the token is the first v whose running sum of u exceeds
// theta = floor(r * S / 2^64), S = sum_v u_v. A row with no finite value
// gives token 0. Integer sums make the draw exact and order-free.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Inclusive prefix sum of a uint64 over the 64 lanes of a wave.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((unsigned int)v, (unsigned int)o, 64);
    const uint32_t hi = __shfl_up((unsigned int)(v >> 32), (unsigned int)o, 64);
    if (lane >= o) v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// Eight consecutive row values as raw bits (bf16: four dwords, f32: eight).
template <typename IN_T>
struct Unit8 {
  uint32_t w[sizeof(IN_T) * 4];
};

template <typename IN_T>
__device__ __forceinline__ void unit_load(const IN_T* row, int u, Unit8<IN_T>& r) {
  const uint4* p = reinterpret_cast<const uint4*>(row) + (size_t)u * (sizeof(IN_T) / 2);
#pragma unroll
  for (int h = 0; h < (int)sizeof(IN_T) / 2; ++h) {
    const uint4 q = p[h];
    r.w[4 * h] = q.x;
    r.w[4 * h + 1] = q.y;
    r.w[4 * h + 2] = q.z;
    r.w[4 * h + 3] = q.w;
  }
}

// Rows whose start is not 16-byte aligned: element by element; -inf past the
// row's end.
template <typename IN_T>
__device__ __forceinline__ void unit_load_scalar(const IN_T* row, int u, int V, Unit8<IN_T>& r) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = u * 8 + k;
    if constexpr (sizeof(IN_T) == 2) {
      const uint32_t bits = e < V ? reinterpret_cast<const uint16_t*>(row)[e] : 0xFF80u;
      if (k & 1) r.w[k >> 1] |= bits << 16;
      else r.w[k >> 1] = bits;
    } else {
      r.w[k] = e < V ? reinterpret_cast<const uint32_t*>(row)[e] : 0xFF800000u;
    }
  }
}

template <typename IN_T>
__device__ __forceinline__ void unit_fill_neg_inf(Unit8<IN_T>& r) {
#pragma unroll
  for (int h = 0; h < (int)sizeof(IN_T) * 4; ++h) r.w[h] = sizeof(IN_T) == 2 ? 0xFF80FF80u : 0xFF800000u;
}

// Value k of a unit as stored (bf16 widened to fp32 exactly).
template <typename IN_T>
__device__ __forceinline__ float unit_raw(const Unit8<IN_T>& r, int k) {
  if constexpr (sizeof(IN_T) == 2)
    return (k & 1) ? __uint_as_float(r.w[k >> 1] & 0xFFFF0000u) : __uint_as_float(r.w[k >> 1] << 16);
  else
    return __uint_as_float(r.w[k]);
}

// Value k as the sampling value x = fp32(raw * inv_tau) (TAU1: inv_tau is 1,
// the product is the value itself); SAN: NaN and +inf ranked as -inf. Rows
// without NaN, +inf or an overflowing product need no SAN.
template <typename IN_T, bool TAU1, bool SAN>
__device__ __forceinline__ float unit_x(const Unit8<IN_T>& r, int k, float inv_tau) {
  float v = unit_raw(r, k);
  if constexpr (!TAU1) v = v * inv_tau;
  if constexpr (SAN) v = (v < INFINITY) ? v : -INFINITY;
  return v;
}

// Maximum of the stored values, and whether any is NaN or +inf.
template <typename IN_T>
__device__ __forceinline__ float unit_max_raw(const Unit8<IN_T>& r, float acc, bool& bad) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float v = unit_raw(r, k);
    bad |= !(v < INFINITY);
    acc = fmaxf(acc, v);
  }
  return acc;
}

template <typename IN_T, bool TAU1>
__device__ __forceinline__ float unit_max(const Unit8<IN_T>& r, float inv_tau, float acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc = fmaxf(acc, unit_x<IN_T, TAU1, true>(r, k, inv_tau));
  return acc;
}

// Replaces every value whose product with inv_tau is NaN or +inf by -inf, in
// place: afterwards the unsanitised weights are the sanitised ones.
template <typename IN_T, bool TAU1>
__device__ __forceinline__ void unit_sanitize(Unit8<IN_T>& r, float inv_tau) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float x = unit_raw(r, k);
    if constexpr (!TAU1) x = x * inv_tau;
    if (!(x < INFINITY)) {
      if constexpr (sizeof(IN_T) == 2)
        r.w[k >> 1] = (k & 1) ? ((r.w[k >> 1] & 0xFFFFu) | 0xFF800000u)
                              : ((r.w[k >> 1] & 0xFFFF0000u) | 0xFF80u);
      else
        r.w[k] = 0xFF800000u;
    }
  }
}

// Sum of the unit's eight fixed-point weights (each <= 2^44: exact in fp64).
template <typename IN_T, bool TAU1, bool SAN>
__device__ __forceinline__ double unit_sum(const Unit8<IN_T>& r, float m, float inv_tau) {
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += exp_fixed(unit_x<IN_T, TAU1, SAN>(r, k, inv_tau) - m);
  return s;
}

constexpr int kSampleBlock = 1024;
constexpr int kSampleWaves = kSampleBlock / 64;
constexpr int kSampleBatch = 4;  // units per lane per round trip when streamed

// One workgroup of 1024 threads per (request, node) row; rows >= num_nodes
// get -1. The row is cut into units of eight values; wave w owns the
// contiguous units [64 C w, 64 C (w + 1)) and lane l of it the units
// 64 C w + 64 j + l (j < C), so every load is a coalesced 1 KiB (bf16) per
// wave and the token order is (wave, slot j, lane, element). CH > 0: the
// row stays in registers (C = CH units per lane) between the maximum, the
// sums and the search; CH == 0: it is streamed (C = chs) and read again.
// AL: rows start 16-byte aligned and V % 8 == 0 (whole-unit vector loads).
// TAU1: inv_tau == 1.
// The maximum is taken over the stored values and scaled once: rounding is
// monotone, so fp32(max raw * inv_tau) is the maximum of the products when
// no value is NaN or +inf and that product is finite; otherwise the exact
// maximum of the sanitised products is taken in a second pass, and the sums
// sanitise too. The search: the wave whose range of the running sum holds
// theta walks its slots j with one wave sum each, then the lane (inclusive
// wave scan) and the value; sums are integers, so the result is that of a
// scan in token order.
template <typename IN_T, int CH, bool AL, bool TAU1>
__global__ __launch_bounds__(kSampleBlock) void k_sample(AcceptArgs a, float inv_tau,
                                                         uint64_t seed, uint64_t offset, int chs,
                                                         int32_t* tgt) {
  __shared__ float s_m[kSampleWaves], s_m2[kSampleWaves];
  __shared__ uint32_t s_bad[kSampleWaves];
  __shared__ uint64_t s_w[kSampleWaves];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T, V = a.V;
  const int rowi = blockIdx.x;
  const int b = rowi / T, i = rowi - b * T;
  if (i >= min(a.num_nodes[b], T)) {
    if (tid == 0) tgt[rowi] = -1;
    return;
  }
  const IN_T* row = static_cast<const IN_T*>(a.target_logits) + (size_t)rowi * V;
  const int nunit = (V + 7) >> 3;
  const int C = CH > 0 ? CH : chs;
  const int ubase = wid * 64 * C + lane;
  // loads always address a unit of the row (clamped index) and are replaced
  // by -inf past its end, so that they issue without branches
  auto fetch = [&](int j, Unit8<IN_T>& r) {
    const int u = j < C ? ubase + 64 * j : nunit;  // slots past C: -inf
    const int uc = min(u, nunit - 1);
    if constexpr (AL) unit_load(row, uc, r);
    else unit_load_scalar(row, uc, V, r);
    if (u >= nunit) unit_fill_neg_inf(r);
  };
  Unit8<IN_T> buf[CH > 0 ? CH : kSampleBatch];
  if constexpr (CH > 0) {
#pragma unroll
    for (int j = 0; j < CH; ++j) fetch(j, buf[j]);
  }
  // the uniform, computed while the loads are in flight
  uint32_t c[4] = {(uint32_t)i, (uint32_t)b, (uint32_t)offset, (uint32_t)(offset >> 32)};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t r = ((uint64_t)c[1] << 32) | c[0];
  // ---- maximum of the stored values
  float lmax = -INFINITY;
  bool bad = false;
  if constexpr (CH > 0) {
#pragma unroll
    for (int j = 0; j < CH; ++j) lmax = unit_max_raw(buf[j], lmax, bad);
  } else {
    for (int j0 = 0; j0 < C; j0 += kSampleBatch) {
#pragma unroll
      for (int q = 0; q < kSampleBatch; ++q) fetch(j0 + q, buf[q]);
#pragma unroll
      for (int q = 0; q < kSampleBatch; ++q) lmax = unit_max_raw(buf[q], lmax, bad);
    }
  }
  if constexpr (CH > 0) {
    // keep only the packed bits live across the barrier: the values are
    // unpacked again for the sums (fewer registers than 8 floats per unit)
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int h = 0; h < (int)sizeof(IN_T) * 4; ++h) asm volatile("" : "+v"(buf[j].w[h]));
  }
  const float wm = wave_max_dpp(lmax);
  const uint64_t wbad = __ballot(bad);
  if (lane == 0) {
    s_m[wid] = wm;
    s_bad[wid] = wbad != 0;
  }
  __syncthreads();
  float m = s_m[0];
  uint32_t anybad = s_bad[0];
#pragma unroll
  for (int w = 1; w < kSampleWaves; ++w) {
    m = fmaxf(m, s_m[w]);
    anybad |= s_bad[w];
  }
  if constexpr (!TAU1) m = m * inv_tau;
  const bool slow = anybad != 0 || !(m < INFINITY);  // block-uniform
  if (slow) {
    // exact maximum of the sanitised products (rows in registers are
    // sanitised in place first, so that the sums below need no check)
    float l2 = -INFINITY;
    if constexpr (CH > 0) {
      bool unused = false;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        unit_sanitize<IN_T, TAU1>(buf[j], inv_tau);
        l2 = unit_max_raw(buf[j], l2, unused);
      }
      if constexpr (!TAU1) l2 = l2 * inv_tau;
    } else {
      for (int j0 = 0; j0 < C; j0 += kSampleBatch) {
#pragma unroll
        for (int q = 0; q < kSampleBatch; ++q) fetch(j0 + q, buf[q]);
#pragma unroll
        for (int q = 0; q < kSampleBatch; ++q) l2 = unit_max<IN_T, TAU1>(buf[q], inv_tau, l2);
      }
    }
    const float w2 = wave_max_dpp(l2);
    if (lane == 0) s_m2[wid] = w2;
    __syncthreads();
    m = s_m2[0];
#pragma unroll
    for (int w = 1; w < kSampleWaves; ++w) m = fmaxf(m, s_m2[w]);
  }
  if (m == -INFINITY) {  // no finite value: token 0
    if (tid == 0) tgt[rowi] = 0;
    return;
  }
  // ---- the weights' sums: per slot and lane (kept for the search), per
  // thread, per wave, whole row
  constexpr int NS = CH > 0 ? CH : 1;
  double su[NS];
  uint64_t tsum = 0;
  if constexpr (CH > 0) {
    double ts = 0.0;  // at most 8 * CH <= 256 weights of <= 2^44: exact
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      su[j] = unit_sum<IN_T, TAU1, false>(buf[j], m, inv_tau);
      ts += su[j];
    }
    tsum = (uint64_t)ts;
  } else {
    for (int j0 = 0; j0 < C; j0 += kSampleBatch) {
#pragma unroll
      for (int q = 0; q < kSampleBatch; ++q) fetch(j0 + q, buf[q]);
      double ts = 0.0;
      if (slow) {
#pragma unroll
        for (int q = 0; q < kSampleBatch; ++q) ts += unit_sum<IN_T, TAU1, true>(buf[q], m, inv_tau);
      } else {
#pragma unroll
        for (int q = 0; q < kSampleBatch; ++q) ts += unit_sum<IN_T, TAU1, false>(buf[q], m, inv_tau);
      }
      tsum += (uint64_t)ts;
    }
  }
  const uint64_t wsum = wave_sum_u64_dpp(tsum);
  if (lane == 0) s_w[wid] = wsum;
  __syncthreads();
  uint64_t S = 0, pre = 0;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) {
    const uint64_t v = s_w[w];
    if (w < wid) pre += v;
    S += v;
  }
  const uint64_t theta = __umul64hi(r, S);
  // exactly one wave holds theta (0 <= theta < S)
  if (!(pre <= theta && theta < pre + wsum)) return;
  // ---- the slot (one wave sum per slot, in order), then the lane and value;
  // weights are recomputed sanitised (equal to the unsanitised ones when no
  // value needs it)
  uint64_t run = pre, sstar = 0;
  int jstar = -1;
  Unit8<IN_T> t;
  if constexpr (CH > 0) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (jstar < 0) {
        const uint64_t sj = (uint64_t)su[j];
        const uint64_t tj = wave_sum_u64_dpp(sj);
        if (theta < run + tj) {
          jstar = j;
          sstar = sj;
        } else {
          run += tj;
        }
      }
    }
  } else {
    for (int j0 = 0; j0 < C && jstar < 0; j0 += kSampleBatch) {
#pragma unroll
      for (int q = 0; q < kSampleBatch; ++q) fetch(j0 + q, buf[q]);
#pragma unroll
      for (int q = 0; q < kSampleBatch; ++q) {
        if (jstar < 0) {
          const uint64_t sj = (uint64_t)unit_sum<IN_T, TAU1, true>(buf[q], m, inv_tau);
          const uint64_t tj = wave_sum_u64_dpp(sj);
          if (theta < run + tj) {
            jstar = j0 + q;
            sstar = sj;
            t = buf[q];
          } else {
            run += tj;
          }
        }
      }
    }
  }
  jstar = max(jstar, 0);  // found unless the sums disagree; keeps indexes in the row
  const uint64_t incl = wave_incl_scan_u64(sstar, lane);
  uint64_t acc = run + incl - sstar;
  int tok = -1;
  if (acc <= theta && theta < acc + sstar) {
    if constexpr (CH > 0 && CH <= 8) {
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if (j == jstar) t = buf[j];
    } else if constexpr (CH > 0) {
      fetch(jstar, t);  // one unit of the row, read again by this lane only
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc += (uint64_t)exp_fixed(unit_x<IN_T, TAU1, true>(t, k, inv_tau) - m);
      if (tok < 0 && acc > theta) tok = (ubase + 64 * jstar) * 8 + k;
    }
  }
  const uint64_t found = __ballot(tok >= 0);
  const int first = found ? (int)__builtin_ctzll(found) : 0;
  const int y = __builtin_amdgcn_readlane(tok, first);
  if (lane == 0) tgt[rowi] = max(y, 0);
}

template <typename IN_T>
hipError_t launch_logits(const AcceptArgs& a, const AcceptWork& w, hipStream_t st) {
  const bool vec = (reinterpret_cast<uintptr_t>(a.target_logits) % 16 == 0) &&
                   ((size_t)a.V * sizeof(IN_T)) % 16 == 0;
  dim3 grid(a.batch * a.T * w.S2);
  const int cv = (int)(((size_t)a.V * sizeof(IN_T) / 16 + w.S2 - 1) / w.S2);  // vectors per chunk
  if (!vec)
    hipLaunchKernelGGL((k_argmax<IN_T, 256, false, 1>), grid, dim3(256), 0, st, a, w.S2, w.pv, w.pidx);
  else if (cv >= 8 * 256)
    hipLaunchKernelGGL((k_argmax<IN_T, 256, true, 8>), grid, dim3(256), 0, st, a, w.S2, w.pv, w.pidx);
  else
    hipLaunchKernelGGL((k_argmax<IN_T, 256, true, 2>), grid, dim3(256), 0, st, a, w.S2, w.pv, w.pidx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T <= 256)
    hipLaunchKernelGGL((k_walk<false, 256>), dim3(a.batch), dim3(256), 0, st, a, w.S2, w.pv, w.pidx);
  else
    hipLaunchKernelGGL((k_walk<false, 1024>), dim3(a.batch), dim3(1024), 0, st, a, w.S2, w.pv, w.pidx);
  return hipGetLastError();
}

}  // namespace

// Chunks per target row: enough workgroups (about 512) to fill the chip when
// the batch has few tree nodes, at most 16.
int accept_splits(int batch, int T) {
  const long long rows = (long long)batch * T;
  return (int)std::min<long long>(16, std::max<long long>(1, (512 + rows - 1) / rows));
}

size_t accept_workspace_bytes(int batch, int T) {
  const size_t parts = (size_t)batch * T * accept_splits(batch, T);
  return 2 * align_up(parts * 4, 256);
}

AcceptWork accept_carve(void* ws, int batch, int T) {
  AcceptWork w;
  w.S2 = accept_splits(batch, T);
  const size_t parts = (size_t)batch * T * w.S2;
  w.pv = reinterpret_cast<float*>(ws);
  w.pidx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(parts * 4, 256));
  return w;
}

template <typename IN_T, bool TAU1>
void launch_sample_rows(const AcceptArgs& a, float inv_tau, uint64_t seed, uint64_t offset,
                        int32_t* tgt, hipStream_t st) {
  const int nunit = (a.V + 7) / 8;
  const int per = (nunit + kSampleBlock - 1) / kSampleBlock;
  const bool al = (a.V % 8 == 0) && (reinterpret_cast<uintptr_t>(a.target_logits) % 16 == 0);
  const dim3 grid(a.batch * a.T), block(kSampleBlock);
#define DDT_SAMPLE(CHV, ALV)                                                                    \
  hipLaunchKernelGGL((k_sample<IN_T, CHV, ALV, TAU1>), grid, block, 0, st, a, inv_tau, seed, \
                     offset, per, tgt)
  if (!al) DDT_SAMPLE(0, false);
  else if (per <= 1) DDT_SAMPLE(1, true);
  else if (per <= 2) DDT_SAMPLE(2, true);
  else if (per <= 4) DDT_SAMPLE(4, true);
  else if (per <= 8) DDT_SAMPLE(8, true);
  else {
    // past 12 units per lane a row in registers leaves one workgroup per CU
    // (loads, sums and search in series); streamed rows run two per CU
    if constexpr (sizeof(IN_T) == 2) {
      if (per <= 12) DDT_SAMPLE(12, true);
      else DDT_SAMPLE(0, true);
    } else {
      DDT_SAMPLE(0, true);
    }
  }
#undef DDT_SAMPLE
}

hipError_t launch_accept_sample(const AcceptArgs& a, float inv_tau, uint64_t seed,
                                uint64_t offset, int32_t* tgt, hipStream_t st) {
  const bool one = inv_tau == 1.0f;
  if (a.dtype == 0) {
    if (one) launch_sample_rows<uint16_t, true>(a, inv_tau, seed, offset, tgt, st);
    else launch_sample_rows<uint16_t, false>(a, inv_tau, seed, offset, tgt, st);
  } else {
    if (one) launch_sample_rows<float, true>(a, inv_tau, seed, offset, tgt, st);
    else launch_sample_rows<float, false>(a, inv_tau, seed, offset, tgt, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AcceptArgs w = a;
  w.target_logits = nullptr;
  w.target_ids = tgt;
  w.target_argmax = nullptr;
  if (a.T <= 256)
    hipLaunchKernelGGL((k_walk<true, 256>), dim3(a.batch), dim3(256), 0, st, w, 0, nullptr, nullptr);
  else
    hipLaunchKernelGGL((k_walk<true, 1024>), dim3(a.batch), dim3(1024), 0, st, w, 0, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& a, const AcceptWork& w, hipStream_t st) {
  if (!a.target_logits) {
    if (a.T <= 256)
      hipLaunchKernelGGL((k_walk<true, 256>), dim3(a.batch), dim3(256), 0, st, a, 0, nullptr, nullptr);
    else
      hipLaunchKernelGGL((k_walk<true, 1024>), dim3(a.batch), dim3(1024), 0, st, a, 0, nullptr, nullptr);
    return hipGetLastError();
  }
  if (a.dtype == 0) return launch_logits<uint16_t>(a, w, st);
  return launch_logits<float>(a, w, st);
}

}  // namespace ddt
