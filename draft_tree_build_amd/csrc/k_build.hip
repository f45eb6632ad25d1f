// Draft-tree build on gfx950: per-position log-softmax + top-K (k_rows); the
// best-first tree and its ancestor bitmask follow in k_tree (k_tree.hip).
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, cited as [BDDT <section>].
//
// k_rows: one workgroup per drafter row (request b, position i), or, when
// there are too few rows to fill the chip, one per chunk of a row (k_rows
// with PART, then k_rows_sum). A workgroup streams its row (chunk) from HBM
// once, kept in registers when it fits, and produces the row maximum, the K
// best tokens as candidate words (ranking key, id) and the exact fixed-point
// softmax normaliser (as partial sums, exact in any order). k_tree turns
// these into log-probabilities.
#include <algorithm>

#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

constexpr int kCandMax = 2048;   // candidate buffer for the top-K sort (LDS)
constexpr int kMaxT = 1025;

struct RowShared {
  uint64_t cand[kCandMax];
};

// ------------------------------------------------------------------ input views
template <typename IN_T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static float scalar(const uint16_t* p, int i) { return bf16_to_float(p[i]); }
  template <class F>
  __device__ __forceinline__ static void unpack(const uint4& r, int base, F&& f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f(base + 2 * j, __uint_as_float(w[j] << 16));
      f(base + 2 * j + 1, __uint_as_float(w[j] & 0xFFFF0000u));
    }
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ __forceinline__ static float scalar(const float* p, int i) { return p[i]; }
  template <class F>
  __device__ __forceinline__ static void unpack(const uint4& r, int base, F&& f) {
    f(base + 0, __uint_as_float(r.x));
    f(base + 1, __uint_as_float(r.y));
    f(base + 2, __uint_as_float(r.z));
    f(base + 3, __uint_as_float(r.w));
  }
};

// A drafter row as seen by one thread. CH > 0: the thread's 16-byte vectors
// c*BLOCK + tid (c < CH) are held in registers; CH == 0: vectors re-read per
// pass; CH < 0: scalar elements (any alignment). Elements are visited in
// increasing token id per thread; chunk c covers ids in a contiguous range.
template <typename IN_T, int BLOCK, int CH>
struct RowView {
  static constexpr int EPV = Elem<IN_T>::kPerVec;
  const IN_T* row;  // first element of the row (chunk)
  int V;            // elements in the row (chunk)
  int nvec;
  int id0;          // token id of element 0
  uint4 reg[CH > 0 ? CH : 1];

  __device__ __forceinline__ void load(int tid) {
    if constexpr (CH > 0) {
      const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        // clamped, unconditional loads: all CH requests are in flight at once;
        // vectors past the row end are never visited
        const int vi = min(c * BLOCK + tid, nvec - 1);
        reg[c] = p[vi];
      }
    }
  }
  // Opaque register barrier between passes: keeps the compiler from caching
  // unpacked values of one pass for the next (which would hold every element
  // of the row in fp32 and spill).
  __device__ __forceinline__ void fence() {
    if constexpr (CH > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        asm volatile("" : "+v"(reg[c].x), "+v"(reg[c].y), "+v"(reg[c].z), "+v"(reg[c].w));
    }
  }
  __device__ __forceinline__ int num_chunks() const {
    if constexpr (CH < 0) return (V + BLOCK - 1) / BLOCK;
    return (nvec + BLOCK - 1) / BLOCK;
  }
  // Chunk c straight from memory (used by the rare exact fallback only, so
  // that the register copy is never indexed by a runtime chunk number).
  template <class F>
  __device__ __forceinline__ void visit_chunk(int c, int tid, F&& f) const {
    if constexpr (CH >= 0) {
      int vi = c * BLOCK + tid;
      if (vi < nvec) Elem<IN_T>::unpack(reinterpret_cast<const uint4*>(row)[vi], id0 + vi * EPV, f);
    } else {
      int v = c * BLOCK + tid;
      if (v < V) f(id0 + v, Elem<IN_T>::scalar(row, v));
    }
  }
  template <class F>
  __device__ __forceinline__ void visit_mem(int tid, F&& f) const {
    const int nc = num_chunks();
    for (int c = 0; c < nc; ++c) visit_chunk(c, tid, f);
  }
  template <class F>
  __device__ __forceinline__ void visit(int tid, F&& f) const {
    if constexpr (CH > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        int vi = c * BLOCK + tid;
        if (vi < nvec) Elem<IN_T>::unpack(reg[c], id0 + vi * EPV, f);
      }
    } else {
      const int nc = num_chunks();
      for (int c = 0; c < nc; ++c) visit_chunk(c, tid, f);
    }
  }
};

// ------------------------------------------------------------------ block helpers
template <int BLOCK>
__device__ float block_max(float v, float* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < BLOCK / 64; ++w) r = fmaxf(r, scratch[w]);
  return r;
}
template <int BLOCK>
__device__ int block_or(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < BLOCK / 64; ++w) r |= scratch[w];
  return r;
}
template <int BLOCK>
__device__ int block_sum(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < BLOCK / 64; ++w) r += scratch[w];
  return r;
}
template <int BLOCK>
__device__ uint64_t block_sum_u64(uint64_t v, uint64_t* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  uint64_t r = 0;
  for (int w = 0; w < BLOCK / 64; ++w) r += scratch[w];
  return r;
}
// Exclusive prefix sum over the block (thread order); returns the block total.
template <int BLOCK>
__device__ int block_exclusive_scan(int v, int* excl, int* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = wave_inclusive_scan(v, lane);
  __syncthreads();
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < BLOCK / 64; ++w) {
    int s = scratch[w];
    if (w < wid) before += s;
    total += s;
  }
  *excl = before + inc - v;
  return total;
}

// Bitonic sort of s[0..P) into descending order; P a power of two.
template <int BLOCK>
__device__ void bitonic_desc(uint64_t* s, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += BLOCK) {
        int a = 2 * i - (i & (j - 1));
        int b = a + j;
        bool desc = (a & k) == 0;
        uint64_t x = s[a], y = s[b];
        if ((x < y) == desc) {
          s[a] = y;
          s[b] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Number of words in s[0..n) (LDS, n >= 1) greater than w. Sixteen reads
// are issued before the first compare so that LDS latency is paid once per
// sixteen words; indexes past the end re-read s[n-1] and are not counted.
__device__ __forceinline__ int count_greater(const uint64_t* s, int n, uint64_t w) {
  int c = 0;
  for (int j = 0; j < n; j += 16) {
    uint64_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = s[min(j + u, n - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u) c += (j + u < n && v[u] > w) ? 1 : 0;
  }
  return c;
}

// Candidate word for the top-K sort: larger = better = (x desc, id asc).
__device__ __forceinline__ uint64_t cand_word(uint32_t key, int id) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// ------------------------------------------------------------------ the kernels
// PART = false: one workgroup per row; writes the row's K best candidate
// words (sorted, best first), its maximum, status bits and fixed-point sum.
// PART = true: one workgroup per chunk s of row r (S chunks of cv vectors);
// writes the chunk's K best words, maximum and status bits; k_rows_sum then
// adds the chunk sums and merges the chunk candidates.
template <typename IN_T, int BLOCK, int CH, bool GENERAL, bool PART>
__global__ __launch_bounds__(BLOCK) void k_rows(BuildArgs a, RowPlan pl) {
  constexpr int NW = BLOCK / 64;
  __shared__ RowShared sm_row;
  __shared__ float red_f[NW];
  __shared__ int red_i[16];
  __shared__ uint32_t red_t[NW];
  __shared__ uint64_t red_u[NW];
  __shared__ int red_c[NW];
  __shared__ int s_cnt;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = PART ? (int)blockIdx.x / pl.S : (int)blockIdx.x;
  const int sidx = PART ? (int)blockIdx.x - r * pl.S : 0;
  const int K = a.K;
  const int mode = GENERAL ? a.mode : 0;
  const float inv_tau = a.inv_tau;

  using View = RowView<IN_T, BLOCK, CH>;
  View view;
  view.row = reinterpret_cast<const IN_T*>(a.logits) + (size_t)r * a.V;
  view.V = a.V;
  view.nvec = a.V / View::EPV;
  view.id0 = 0;
  if (PART) {
    const int v0 = sidx * pl.cv;
    view.nvec = min(pl.cv, view.nvec - v0);
    view.V = view.nvec * View::EPV;
    view.id0 = v0 * View::EPV;
    view.row += view.id0;
  }
  view.load(tid);

  auto xval = [&](float raw) __attribute__((always_inline)) -> float {  // ranking value before sanitising
    float x = raw;
    if (GENERAL && mode == 1) x = x * inv_tau;
    return x;
  };

  // ---- pass 1: maximum, non-finite flag, per-thread maximum key
  float tmax = -INFINITY;
  int tflag = 0;
  bool has = false;
  view.visit(tid, [&](int, float raw) __attribute__((always_inline)) {
    float x = xval(raw);
    const bool bad = __builtin_amdgcn_classf(x, 0x203);  // NaN or +inf
    tflag |= bad ? 1 : 0;
    x = bad ? -INFINITY : x;
    tmax = fmaxf(tmax, x);
    has = true;
  });

  // ---- per wave: maximum, status bits, and the K-th largest of its lanes'
  //      maxima (each a distinct element of the row); the largest of the
  //      waves' K-th values is a lower bound t0 for the row's K-th largest key
  {
    const float wm = wave_max_dpp(tmax);
    const uint32_t wf = wave_or_dpp((uint32_t)tflag);
    const uint32_t wt = wave_kth_largest(has ? float_order(tmax) : 0u, K);
    if (lane == 0) {
      red_f[wid] = wm;
      red_i[wid] = (int)wf;
      red_t[wid] = wt;
    }
  }
  __syncthreads();
  float m = red_f[0];
  int flags = red_i[0];
  uint32_t t0 = red_t[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    m = fmaxf(m, red_f[w]);
    flags |= red_i[w];
    t0 = max(t0, red_t[w]);
  }
  // every element with key >= t0 compares >= t0f (a superset when t0f is
  // +0, which also admits -0: harmless, the sort below uses exact keys)
  const float t0f = t0 == 0u ? -INFINITY : order_to_float(t0);

  auto key_of = [&](float raw) __attribute__((always_inline)) -> uint32_t {
    float x = xval(raw);
    x = ((x != x) || (x == INFINITY)) ? -INFINITY : x;
    return float_order(x);
  };
  // candidates go to the wave's own segment of the buffer, at positions
  // from the ballot (no atomics); wcnt is the wave's running count
  constexpr int SEG = kCandMax / NW;
  uint64_t* const seg = sm_row.cand + wid * SEG;
  int wcnt = 0;
  auto take = [&](int id, float xs) __attribute__((always_inline)) {
    const bool hit = xs >= t0f;
    const uint64_t bal = __ballot(hit);
    if (bal != 0ull) {
      const int pos = wcnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (hit && pos < SEG) seg[pos] = cand_word(float_order(xs), id);
      wcnt += __popcll(bal);
    }
  };

  // ---- pass 2: candidates; without a split also the exact fixed-point
  //      normaliser S = sum_v rint(2^44 E(x_v - m))
  double acc = 0.0;
  const bool finite_m = m != -INFINITY;
  view.fence();
  if (flags == 0 && finite_m && !(GENERAL && mode == 2)) {
    // no NaN or +inf in the row: values need no sanitising
    view.visit(tid, [&](int id, float raw) __attribute__((always_inline)) {
      const float x = xval(raw);
      take(id, x);
      if (!PART) acc += exp_fixed(x - m);
    });
  } else {
    // (rows with NaN / +inf, argmax mode): on long rows this pass re-reads
    // memory, so that the register copy is visited by one unrolled loop only
    auto general = [&](int id, float raw) __attribute__((always_inline)) {
      const float x = xval(raw);
      const float xs = ((x != x) || (x == INFINITY)) ? -INFINITY : x;
      take(id, xs);
      if (!PART) {
        float d = (GENERAL && mode == 2) ? ((xs == m) ? 0.0f : -INFINITY) : (xs - m);
        d = finite_m ? d : -INFINITY;
        acc += exp_fixed(d);
      }
    };
    if constexpr (CH > 8) {
      view.visit_mem(tid, general);
    } else {
      view.visit(tid, general);
    }
  }
  if (lane == 0) red_c[wid] = wcnt;
  __syncthreads();
  int cnt[NW];
  int ncand = 0, maxc = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    cnt[w] = red_c[w];
    ncand += cnt[w];
    maxc = max(maxc, cnt[w]);
  }
  const bool over = maxc > SEG;
  uint64_t* out = PART ? a.part_cand + ((size_t)r * pl.S + sidx) * K : a.row_cand + (size_t)r * K;
  if (!over && ncand <= BLOCK) {
    // rank selection: candidate words are distinct (ids differ), so the
    // number of larger words is the position in descending order
    if (tid < ncand) {
      int i = tid, sw = 0;
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) {
        if (sw == w && i >= cnt[w]) {
          i -= cnt[w];
          sw = w + 1;
        }
      }
      const uint64_t word = sm_row.cand[sw * SEG + i];
      // the segments are read side by side, U words of each per round trip
      constexpr int U = NW > 4 ? 4 : 8;
      int rank = 0;
      for (int j = 0; j < maxc; j += U) {
        uint64_t v[NW][U];
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int u = 0; u < U; ++u) v[w][u] = sm_row.cand[w * SEG + min(j + u, max(cnt[w] - 1, 0))];
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int u = 0; u < U; ++u) rank += (j + u < cnt[w] && v[w][u] > word) ? 1 : 0;
      }
      if (rank < K) out[rank] = word;
    } else if (tid < K) {
      out[tid] = 0;  // fewer elements than K: padding below every real word
    }
  } else {
    int nsort;
    if (!over) {
      // more candidates than threads: zero the segment tails (0 is below
      // every real word) and sort the whole buffer
#pragma unroll
      for (int w = 0; w < NW; ++w)
        for (int i = cnt[w] + tid; i < SEG; i += BLOCK) sm_row.cand[w * SEG + i] = 0;
      nsort = kCandMax;
    } else {
      // Exact fallback (rows with very many near-top ties): find the K-th
      // largest key bit by bit, then keep the keys above it and the lowest
      // ids among the keys equal to it.
      uint32_t t = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        int cnt = 0;
        view.visit_mem(tid, [&](int, float raw) __attribute__((always_inline)) { cnt += key_of(raw) >= c ? 1 : 0; });
        if (block_sum<BLOCK>(cnt, red_i) >= K) t = c;
      }
      int gt = 0;
      view.visit_mem(tid, [&](int, float raw) __attribute__((always_inline)) { gt += key_of(raw) > t ? 1 : 0; });
      const int ngt = block_sum<BLOCK>(gt, red_i);
      if (tid == 0) s_cnt = 0;
      __syncthreads();
      view.visit_mem(tid, [&](int id, float raw) __attribute__((always_inline)) {
        uint32_t kk = key_of(raw);
        if (kk > t) sm_row.cand[atomicAdd(&s_cnt, 1)] = cand_word(kk, id);
      });
      const int need = K - ngt;
      int base = 0;
      const int nc = view.num_chunks();
      for (int c = 0; c < nc && base < need; ++c) {
        int local = 0;
        view.visit_chunk(c, tid, [&](int, float raw) __attribute__((always_inline)) { local += key_of(raw) == t ? 1 : 0; });
        int excl;
        const int total = block_exclusive_scan<BLOCK>(local, &excl, red_i);
        int j = 0;
        view.visit_chunk(c, tid, [&](int id, float raw) __attribute__((always_inline)) {
          if (key_of(raw) == t) {
            if (base + excl + j < need) sm_row.cand[atomicAdd(&s_cnt, 1)] = cand_word(t, id);
            ++j;
          }
        });
        base += total;
      }
      __syncthreads();
      nsort = K;
    }
    int P = 2;
    while (P < max(nsort, K)) P <<= 1;
    for (int i = nsort + tid; i < P; i += BLOCK) sm_row.cand[i] = 0;  // 0: below every real word
    __syncthreads();
    bitonic_desc<BLOCK>(sm_row.cand, P);
    if (tid < K) out[tid] = sm_row.cand[tid];
  }

  // ---- the row's (chunk's) maximum, status bits and fixed-point sum
  if (PART) {
    if (tid == 0) {
      const int q = r * pl.S + sidx;
      a.part_max[q] = m;
      a.part_flags[q] = flags;
    }
  } else {
    const uint64_t ws = wave_sum_u64_dpp((uint64_t)acc);
    if (lane == 0) red_u[wid] = ws;
    __syncthreads();
    if (tid == 0) {
      uint64_t S = red_u[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) S += red_u[w];
      a.row_max[r] = m;
      a.row_flags[r] = flags | (m == -INFINITY ? 2 : 0);
      a.row_sum[r] = S;
    }
  }
}

// Second stage of a split row. Workgroups [0, rows*S): the fixed-point sum
// of chunk s with the row maximum over all chunks. Workgroups [rows*S,
// rows*S + rows): the merge of row r's S chunk lists (each its chunk's K best
// words, best first) into the row's K best, its maximum and status bits.
template <typename IN_T, int BLOCK, int CH, bool GENERAL>
__global__ __launch_bounds__(BLOCK) void k_rows_sum(BuildArgs a, RowPlan pl) {
  constexpr int NW = BLOCK / 64;
  __shared__ uint64_t red_u[NW];
  __shared__ uint64_t cands[512];
  __shared__ uint64_t s_T;
  __shared__ int s_cnt;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K;
  const int rows = a.batch * a.L;
  if ((int)blockIdx.x >= rows * pl.S) {
    const int r = (int)blockIdx.x - rows * pl.S;
    const int S = pl.S, q0 = r * S, nw = S * K;  // nw <= 512: two words per thread
    const uint64_t* pc = a.part_cand + (size_t)q0 * K;
    const uint64_t w0 = tid < nw ? pc[tid] : 0ull;
    const uint64_t w1 = tid + BLOCK < nw ? pc[tid + BLOCK] : 0ull;
    if (tid == 0) s_cnt = 0;
    if (wid == 0) {
      // threshold T: the K-th largest of the first qf words of every chunk
      // (S * qf >= K distinct words, so at least K words are >= T); lane l
      // holds the l-th of them and counts the larger ones by broadcasts.
      // The chunk maxima and flags are requested together with the words.
      const int qf = (K + S - 1) / S, n1 = S * qf;  // n1 < K + S <= 64
      const uint64_t f = lane < n1 ? pc[(lane / qf) * K + lane % qf] : 0ull;
      const float pmax = lane < S ? a.part_max[q0 + lane] : -INFINITY;
      const uint32_t pfl = lane < S ? (uint32_t)a.part_flags[q0 + lane] : 0u;
      const uint32_t fh = (uint32_t)(f >> 32), flo = (uint32_t)f;
      int rank = 0;
      for (int j = 0; j < n1; ++j) {
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)fh, j) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)flo, j);
        rank += o > f ? 1 : 0;
      }
      const uint64_t hit = __ballot(lane < n1 && rank == K - 1);
      uint64_t T = 0ull;  // no word of rank K-1 (padding words only): keep all
      if (hit != 0ull) {
        const int l = __ffsll((unsigned long long)hit) - 1;
        T = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)fh, l) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)flo, l);
      }
      const float m = wave_max_dpp(pmax);
      const uint32_t fl = wave_or_dpp(pfl);
      if (lane == 0) {
        s_T = T;
        a.row_max[r] = m;
        a.row_flags[r] = (int)fl | (m == -INFINITY ? 2 : 0);
      }
    }
    __syncthreads();
    const uint64_t T = s_T;
    if (w0 >= T && w0 != 0ull) cands[atomicAdd(&s_cnt, 1)] = w0;
    if (w1 >= T && w1 != 0ull) cands[atomicAdd(&s_cnt, 1)] = w1;
    __syncthreads();
    const int nc = s_cnt;
    for (int i = tid; i < max(nc, K); i += BLOCK) {
      if (i < nc) {
        const uint64_t w = cands[i];
        const int rank = count_greater(cands, nc, w);
        if (rank < K) a.row_cand[(size_t)r * K + rank] = w;
      } else {
        a.row_cand[(size_t)r * K + i] = 0;
      }
    }
    return;
  }

  const int r = (int)blockIdx.x / pl.S;
  const int sidx = (int)blockIdx.x - r * pl.S;
  const int mode = GENERAL ? a.mode : 0;
  const float inv_tau = a.inv_tau;

  using View = RowView<IN_T, BLOCK, CH>;
  View view;
  const int v0 = sidx * pl.cv;
  view.nvec = min(pl.cv, a.V / View::EPV - v0);
  view.V = view.nvec * View::EPV;
  view.id0 = v0 * View::EPV;
  view.row = reinterpret_cast<const IN_T*>(a.logits) + (size_t)r * a.V + view.id0;
  view.load(tid);

  // row maximum and status bits over the S chunks (S <= 64: one load per lane)
  const int q0 = r * pl.S;
  const float pmax = lane < pl.S ? a.part_max[q0 + lane] : -INFINITY;
  const uint32_t pfl = lane < pl.S ? (uint32_t)a.part_flags[q0 + lane] : 0u;
  const float m = wave_max_dpp(pmax);
  const uint32_t fl = wave_or_dpp(pfl);

  double acc = 0.0;
  const bool finite_m = m != -INFINITY;
  if (fl == 0 && finite_m && !(GENERAL && mode == 2)) {
    view.visit(tid, [&](int, float raw) __attribute__((always_inline)) {
      float x = raw;
      if (GENERAL && mode == 1) x = x * inv_tau;
      acc += exp_fixed(x - m);
    });
  } else {
    view.visit(tid, [&](int, float raw) __attribute__((always_inline)) {
      float x = raw;
      if (GENERAL && mode == 1) x = x * inv_tau;
      const float xs = ((x != x) || (x == INFINITY)) ? -INFINITY : x;
      float d = (GENERAL && mode == 2) ? ((xs == m) ? 0.0f : -INFINITY) : (xs - m);
      d = finite_m ? d : -INFINITY;
      acc += exp_fixed(d);
    });
  }
  const uint64_t ws = wave_sum_u64_dpp((uint64_t)acc);
  if (lane == 0) red_u[wid] = ws;
  __syncthreads();
  if (tid == 0) {
    uint64_t S = red_u[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) S += red_u[w];
    a.row_sum[(size_t)q0 + sidx] = S;
  }
}

// Standalone ancestor mask of given trees [BDDT Abstract, §4.1].
__global__ __launch_bounds__(256) void k_mask(const int32_t* parents, const int32_t* num_nodes,
                                              int T, uint64_t* mask) {
  __shared__ int32_t par[kMaxT];
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < T; i += 256) par[i] = parents[(size_t)b * T + i];
  __syncthreads();
  const int nn = num_nodes[b];
  const int W = (T + 63) >> 6;
  for (int idx = threadIdx.x; idx < T * W; idx += 256) {
    const int i = idx / W, w = idx - (idx / W) * W;
    uint64_t bits = 0;
    if (i < nn) {
      int j = i;
      int guard = 0;
      while (j >= 64 * w && guard++ <= kMaxT) {
        if (j < 64 * (w + 1)) bits |= 1ull << (j - 64 * w);
        const int pj = par[j];
        j = (pj < j) ? pj : -1;  // malformed input (parent >= child) ends the walk
      }
    }
    mask[((size_t)b * T + i) * W + w] = bits;
  }
}

template <typename IN_T, int BLOCK, int CH>
hipError_t launch_t(const BuildArgs& a, RowPlan pl, hipStream_t st) {
  dim3 grid(a.batch * a.L), block(BLOCK);
  if (a.mode == 0) {
    hipLaunchKernelGGL((k_rows<IN_T, BLOCK, CH, false, false>), grid, block, 0, st, a, pl);
  } else {
    hipLaunchKernelGGL((k_rows<IN_T, BLOCK, CH, true, false>), grid, block, 0, st, a, pl);
  }
  return hipGetLastError();
}

// Split rows: 256 threads per chunk, the chunk's vectors in registers.
template <typename IN_T, int CH>
hipError_t launch_split(const BuildArgs& a, RowPlan pl, hipStream_t st) {
  const int rows = a.batch * a.L;
  dim3 grid(rows * pl.S), grid2(rows * pl.S + rows), block(256);
  if (a.mode == 0) {
    hipLaunchKernelGGL((k_rows<IN_T, 256, CH, false, true>), grid, block, 0, st, a, pl);
    hipLaunchKernelGGL((k_rows_sum<IN_T, 256, CH, false>), grid2, block, 0, st, a, pl);
  } else {
    hipLaunchKernelGGL((k_rows<IN_T, 256, CH, true, true>), grid, block, 0, st, a, pl);
    hipLaunchKernelGGL((k_rows_sum<IN_T, 256, CH, true>), grid2, block, 0, st, a, pl);
  }
  return hipGetLastError();
}

template <typename IN_T>
hipError_t launch_dt(const BuildArgs& a, RowPlan pl, hipStream_t st) {
  constexpr int EPV = Elem<IN_T>::kPerVec;
  if (pl.S > 1) {
    const int ch = (pl.cv + 255) / 256;
    if (ch <= 1) return launch_split<IN_T, 1>(a, pl, st);
    if (ch <= 2) return launch_split<IN_T, 2>(a, pl, st);
    if (ch <= 4) return launch_split<IN_T, 4>(a, pl, st);
    return launch_split<IN_T, 8>(a, pl, st);
  }
  if (!pl.vec_ok) return launch_t<IN_T, 256, -1>(a, pl, st);
  const int nvec = a.V / EPV;
  if (nvec <= 256) return launch_t<IN_T, 256, 1>(a, pl, st);
  const int ch = (nvec + 511) / 512;
  if (ch <= 4) return launch_t<IN_T, 512, 4>(a, pl, st);
  if (ch <= 8) return launch_t<IN_T, 512, 8>(a, pl, st);
  // longer rows are split (plan_rows) unless their chunks would outnumber
  // what the merge holds: those stream from memory
  return launch_t<IN_T, 512, 0>(a, pl, st);
}

}  // namespace

// Rows are split when there are too few of them to give the chip ~512
// workgroups: S chunks of cv >= 256 vectors each (a vector per thread or
// more, and no chunk empty), S <= 32 and S * K <= 512 (the merge holds all
// S * K words in LDS). Rows longer than 8 * 512 vectors are split into chunks
// of at most 2048 vectors (the register-resident split kernels' limit)
// whatever their number: a whole-row kernel holding up to 40 vectors per
// thread runs one workgroup per compute unit, so a row's loads and its
// arithmetic never overlap, while chunk workgroups run several per unit
// (measured with V = 151,936 bf16: 512 rows 82.9 -> 69.8 us, 128 rows
// 40.6 -> 30.9 us, both kernels together).
RowPlan plan_rows(int batch, int L, int V, int K, int esize, bool vec_ok) {
  RowPlan pl{1, 0, vec_ok};
  const int rows = batch * L;
  const int nvec = (int)(((long long)V * esize) / 16);
  if (!vec_ok) return pl;
  const int smax = std::min(32, 512 / K);
  const int s_long = (nvec + 2047) / 2048;  // fewest chunks of <= 2048 vectors
  int S;
  if (rows >= 256) {
    if (nvec <= 8 * 512) return pl;
    S = s_long;
  } else {
    S = std::min(smax, (512 + rows - 1) / rows);
    S = std::min(S, nvec / 256);
    if (nvec > 8 * 512) S = std::max(S, s_long);
  }
  if (S <= 1 || S > smax) return pl;
  pl.S = S;
  pl.cv = (nvec + S - 1) / S;
  if (pl.cv > 8 * 256) pl.S = 1;  // chunk too long for the register-resident split kernels
  return pl;
}

size_t build_workspace_bytes(int batch, int L, int V, int K) {
  // the largest plan over both element sizes (f32 rows have the most vectors)
  const RowPlan p4 = plan_rows(batch, L, V, K, 4, true), p2 = plan_rows(batch, L, V, K, 2, true);
  return build_layout(batch, L, K, std::max(p4.S, p2.S), nullptr, nullptr);
}

size_t build_layout(int batch, int L, int K, int S, void* ws, BuildArgs* a) {
  const size_t rows = (size_t)batch * L;
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return q;
  };
  char* row_cand = take(rows * K * 8);
  char* row_sum = take(rows * S * 8);
  char* row_max = take(rows * 4);
  char* row_flags = take(rows * 4);
  char* part_cand = S > 1 ? take(rows * S * K * 8) : nullptr;
  char* part_max = S > 1 ? take(rows * S * 4) : nullptr;
  char* part_flags = S > 1 ? take(rows * S * 4) : nullptr;
  if (a) {
    a->row_cand = reinterpret_cast<uint64_t*>(row_cand);
    a->row_sum = reinterpret_cast<uint64_t*>(row_sum);
    a->row_max = reinterpret_cast<float*>(row_max);
    a->row_flags = reinterpret_cast<int32_t*>(row_flags);
    a->part_cand = reinterpret_cast<uint64_t*>(part_cand);
    a->part_max = reinterpret_cast<float*>(part_max);
    a->part_flags = reinterpret_cast<int32_t*>(part_flags);
  }
  return off;
}

hipError_t launch_build(BuildArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  const int esize = a.dtype == 0 ? 2 : 4;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) &&
                      ((size_t)a.V * esize) % 16 == 0;
  const RowPlan pl = plan_rows(a.batch, a.L, a.V, a.K, esize, vec_ok);
  if (build_layout(a.batch, a.L, a.K, pl.S, nullptr, nullptr) > ws_bytes) return hipErrorInvalidValue;
  build_layout(a.batch, a.L, a.K, pl.S, ws, &a);
  hipError_t e = (a.dtype == 0) ? launch_dt<uint16_t>(a, pl, st) : launch_dt<float>(a, pl, st);
  if (e != hipSuccess) return e;
  TreeArgs t{};
  t.row_cand = a.row_cand;
  t.row_sum = a.row_sum;
  t.row_max = a.row_max;
  t.row_flags = a.row_flags;
  t.S = pl.S;
  t.mode = a.mode;
  t.root_tokens = a.root_tokens;
  t.L = a.L;
  t.K = a.K;
  t.N = a.N;
  t.tokens = a.tokens;
  t.parents = a.parents;
  t.depths = a.depths;
  t.scores = a.scores;
  t.num_nodes = a.num_nodes;
  t.mask = a.mask;
  t.topk_tok = a.topk_tok;
  t.topk_lp = a.topk_lp;
  t.status = a.status;
  return launch_tree(t, a.batch, st);
}

hipError_t launch_mask(const int32_t* parents, const int32_t* num_nodes, int batch, int T,
                       uint64_t* mask, hipStream_t st) {
  hipLaunchKernelGGL(k_mask, dim3(batch), dim3(256), 0, st, parents, num_nodes, T, mask);
  return hipGetLastError();
}

}  // namespace ddt
