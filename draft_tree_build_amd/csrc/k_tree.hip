// Draft-tree log-probabilities, best-first tree and ancestor bitmask on
// gfx950 (k_tree).
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, cited as [BDDT <section>].
//
// One workgroup per request. The workgroup first turns the row stage's
// candidate words, maxima and fixed-point sums into the top-K tables
// (token, log-probability) per position. Wave 0 then runs the N pops of the best-first
// search [BDDT §4.3, App. A]. The best pending candidates are kept sorted
// across the 64 lanes of the wave (lane j holds the j-th best), so a pop is
// a read of lane 0, and the popped node's two successors are merged in with
// one wave-wide shift per field: no reduction over the frontier per pop.
// Candidates that fall behind the 64 best go to an unsorted overflow list in
// LDS, kept so that every key in it is worse than every key in the lanes;
// when the lanes run dry, the whole workgroup sorts the overflow list and
// its 64 best return to the lanes. Afterwards the workgroup decodes the
// popped keys into the tree arrays and writes the mask rows.
#include <type_traits>

#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

constexpr uint64_t kEmpty = ~0ull;
constexpr int kMaxLK = 64 * 32;
constexpr int kMaxT = 1025;
constexpr int kOverCap = 2048;  // overflow keys: at most kMaxT live, sorted in place
constexpr int kBlock = 256;
constexpr int kShl1 = 0x130;    // DPP wave_shl:1  lane i reads lane i + 1
constexpr int kShr1 = 0x138;    // DPP wave_shr:1  lane i reads lane i - 1

typedef float floatx32 __attribute__((ext_vector_type(32)));

struct TreeShared {
  int32_t tok[kMaxLK];          // top-K tokens per position, [L, K]
  float lp[kMaxLK + 2];         // their log-probabilities (+2: reads past the last row)
  uint64_t nkey[kMaxT + 63];    // key of the candidate that became node i
  union {
    uint64_t over[kOverCap];    // overflow candidates (during the pops)
    int32_t par[kMaxT];         // parents (mask walk, afterwards)
  };
  float rmax[64];               // row maxima
  float rlse[64];               // row log-normalisers
  int cmd;                      // 1: sort the overflow list; 0: pops finished
  int nover;
  int nn;
};

// Candidate key, smaller = popped first: score desc, then depth, parent and
// rank asc [BDDT App. A tie order]. The high word is the score (see tree_pops).
__device__ __forceinline__ uint32_t key_lo(int depth, int parent, int rank) {
  return ((uint32_t)depth << 25) | ((uint32_t)parent << 14) | ((uint32_t)rank << 9);
}
__device__ __forceinline__ uint64_t key64(uint32_t hi, uint32_t lo) {
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t rdlane(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ float rdlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Write the uniform value s into lane `lane` of v.
__device__ __forceinline__ uint32_t wrlane(uint32_t v, uint32_t s, uint32_t lane) {
  asm("v_writelane_b32 %0, %1, m0" : "+v"(v) : "s"(s), "{m0}"(lane));
  return v;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shift(uint32_t fill, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {  // lanes without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Ascending bitonic sort of over[0..count), run by the whole workgroup.
__device__ void sort_over(TreeShared& sh, int count) {
  int P = 2;
  while (P < count) P <<= 1;
  for (int i = count + (int)threadIdx.x; i < P; i += kBlock) sh.over[i] = kEmpty;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += kBlock) {
        const int x = 2 * i - (i & (j - 1));
        const int y = x + j;
        const bool up = (x & k) == 0;
        const uint64_t u = sh.over[x], w = sh.over[y];
        if ((u > w) == up) {
          sh.over[x] = w;
          sh.over[y] = u;
        }
      }
      __syncthreads();
    }
  }
}

// The N pops of one request, run by wave 0 [BDDT §4.3, App. A].
//
// Scores are sums of log-probabilities, so they are <= 0 and never -0; on
// that range the raw float bits order scores in reverse, and the high word
// of a key is the score's bit pattern itself (+0 -> 0, -inf -> 0xFF800000,
// 0xFFFFFFFF marks "no candidate").
//
// A pending candidate is (key, ps): ps is its parent's score. Popping
// candidate (d, p, r) with score s yields
//   sibling (d, p, r+1): score ps + lp[d-1][r+1] (when rank r+1 exists)
//   child (d+1, n, 0):   score s + lp[d][0]
// -- the log-probability table sits in registers (lane d, element k holds
// lp[d][k]), so each is one indexed register move and one lane read --
// and the lane array is rebuilt from the old lanes shifted by -1, 0 or +1
// plus the two new candidates c1 < c2, lane j taking
//   old j+1 if it precedes c1 | c1 | old j if between | c2 | old j-1.
//
// With more than 64 pops to go, candidates behind the 64 lanes are kept in
// the overflow list (every overflow key worse than every lane key). Once the
// occupied lanes are at least the pops still to come, nothing behind them can
// be popped any more: the overflow list is dropped and the simpler loop runs.
// Returns num_nodes (root included); node keys are left in sh.nkey.
constexpr uint32_t kNone = 0xFFFFFFFFu;

template <bool SIB>
__device__ int tree_pops(TreeShared& sh, int L, int K, int N) {
  const int lane = threadIdx.x & 63;
  floatx32 tbl;
#pragma unroll
  for (int k = 0; k < 32; ++k) tbl[k] = (lane < L && k < K) ? sh.lp[lane * K + k] : 0.0f;
  const uint32_t rank_lim = (uint32_t)K << 9;  // rank field limit

  uint32_t Hh = kNone, Hl = kNone, Hps = 0u;
  if (lane == 0) {  // the root's best child: depth 1, parent 0, rank 0
    Hh = __float_as_uint(0.0f + sh.lp[0]);
    Hl = key_lo(1, 0, 0);
    Hps = __float_as_uint(0.0f);
  }
  uint32_t rec_h = 0u, rec_l = 0u;  // popped keys, node i in lane i % 64 (node 0: root)
  int h = 1;
  int nover = 0;
  uint64_t omin = kEmpty;
  int n = 1;

  // One pop; OVER: keep candidates behind the lanes in the overflow list.
  // MODE 0: lanes only; 1: lanes and the overflow list; 2: lanes only,
  // counting the occupied lanes in h (the window cannot overflow yet)
  auto pop = [&](auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool OVER = MODE == 1;
    const uint32_t xh = rdlane(Hh, 0), xl = rdlane(Hl, 0), xps = rdlane(Hps, 0);
    rec_h = wrlane(rec_h, xh, (uint32_t)(n & 63));
    rec_l = wrlane(rec_l, xl, (uint32_t)(n & 63));
    if ((n & 63) == 63) sh.nkey[(n & ~63) + lane] = key64(rec_h, rec_l);
    const int d = (int)(xl >> 25);     // 1..L
    const int dc = d & 63;             // lane of position d (unused when d == L == 64)
    const uint32_t rf = xl & 0x3E00u;  // rank << 9
    const float s = __uint_as_float(xh);
    // sibling: lp[d-1][r+1] is element r+1 of lane d-1 (the index is clamped
    // when rank r+1 does not exist: the value is then unused)
    uint64_t ks = kEmpty;
    if (SIB && rf + 512u < rank_lim) {
      const float lsib = rdlane_f(tbl[min((int)(rf >> 9) + 1, 31)], d - 1);
      ks = key64(__float_as_uint(__uint_as_float(xps) + lsib), xl + 512u);
    }
    // child: lane d of the all-lane sums s + lp[.][0]
    const uint32_t cs = rdlane(__float_as_uint(s + tbl[0]), dc);
    const uint64_t kc = d < L ? key64(cs, ((xl & 0xFE000000u) + 0x02000000u) | ((uint32_t)n << 14))
                              : kEmpty;
    const bool sf = ks < kc;
    uint64_t c1 = sf ? ks : kc, c2 = sf ? kc : ks;
    const uint32_t ps1 = sf ? xps : xh, ps2 = sf ? xh : xps;

    if constexpr (OVER) {
      const bool in1 = c1 < omin, in2 = c2 < omin;
      if (c1 != kEmpty && !in1) {
        if (lane == 0) sh.over[nover] = c1;
        ++nover;
        omin = c1 < omin ? c1 : omin;
      }
      if (c2 != kEmpty && !in2) {
        if (lane == 0) sh.over[nover] = c2;
        ++nover;
      }
      if (!in1) c1 = kEmpty;
      if (!in2) c2 = kEmpty;
      if (in2 && h == 64) {  // 63 + 2 candidates: the 65th joins the overflow list
        const uint64_t Hk = key64(Hh, Hl);
        const uint64_t ev = __ballot(c2 < Hk) ? key64(rdlane(Hh, 63), rdlane(Hl, 63)) : c2;
        if (lane == 0) sh.over[nover] = ev;
        ++nover;
        omin = ev < omin ? ev : omin;
        h -= 1;
      }
      h += (in1 ? 1 : 0) + (in2 ? 1 : 0) - 1;
    }

    if constexpr (MODE == 2) h += (c1 != kEmpty ? 1 : 0) + (c2 != kEmpty ? 1 : 0) - 1;

    // rebuild the lanes
    const uint32_t slh = dpp_shift<kShl1>(kNone, Hh), sll = dpp_shift<kShl1>(kNone, Hl);
    const uint32_t srh = dpp_zero<kShr1>(Hh), srl = dpp_zero<kShr1>(Hl);
    const uint64_t Hk = key64(Hh, Hl);
    const bool a_here = c1 < Hk, b_here = c2 < Hk;            // old j is behind c1 / c2
    const bool a_next = c1 < key64(slh, sll);                 // old j+1 is behind c1
    const bool b_prev = c2 < key64(srh, srl);                 // old j-1 is behind c2
    auto pick = [&](uint32_t sl, uint32_t same, uint32_t sr, uint32_t v1, uint32_t v2)
        __attribute__((always_inline)) -> uint32_t {
      return !a_next ? sl : !a_here ? v1 : !b_here ? same : !b_prev ? v2 : sr;
    };
    Hh = pick(slh, Hh, srh, (uint32_t)(c1 >> 32), (uint32_t)(c2 >> 32));
    Hl = pick(sll, Hl, srl, (uint32_t)c1, (uint32_t)c2);
    Hps = pick(dpp_zero<kShl1>(Hps), Hps, dpp_zero<kShr1>(Hps), ps1, ps2);
  };

  if (N > 64) {
    // While at most 62 lanes are occupied a pop cannot push a candidate
    // behind the lanes (it removes one and adds at most two): the overflow
    // bookkeeping starts only when the window is about to fill.
    for (; n <= N && h <= 62; ++n) {
      if (rdlane(Hh, 0) == kNone) break;
      pop(std::integral_constant<int, 2>{});
    }
    for (; n <= N; ++n) {
      if (h == 0) {
        if (nover == 0) break;  // the tree holds every node the tables allow
        // refill the lanes with the 64 best overflow candidates
        sh.nkey[(n & ~63) + lane] = key64(rec_h, rec_l);
        if (lane == 0) {
          sh.cmd = 1;
          sh.nover = nover;
        }
        __syncthreads();
        sort_over(sh, nover);
        const int take = min(64, nover);
        const uint64_t k = lane < take ? sh.over[lane] : kEmpty;
        Hh = (uint32_t)(k >> 32);
        Hl = (uint32_t)k;
        Hps = 0u;
        if (lane < take) Hps = (uint32_t)(sh.nkey[(Hl >> 14) & 0x7FFu] >> 32);  // parent's score
        for (int i = take + lane; i < nover; i += 64) sh.over[i - take] = sh.over[i];
        nover -= take;
        omin = nover > 0 ? sh.over[0] : kEmpty;
        h = take;
      }
      pop(std::integral_constant<int, 1>{});
      if (h >= N - n) {  // the lanes cover every remaining pop
        ++n;
        break;
      }
    }
  }
  // every remaining pop is served by the lanes; a dry lane array ends the tree
  for (; n <= N; ++n) {
    if (rdlane(Hh, 0) == kNone) break;
    pop(std::integral_constant<int, 0>{});
  }
  sh.nkey[((n - 1) & ~63) + lane] = key64(rec_h, rec_l);
  return n;
}

// One workgroup per request: pops (wave 0, helped by the others for
// overflow sorts), then tree arrays and mask rows [BDDT Abstract, §4.1].
__global__ __launch_bounds__(kBlock) void k_tree(TreeArgs a) {
  __shared__ TreeShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x;
  const int K = a.K, L = a.L, S = a.S;
  const int LK = L * K;
  const size_t r0 = (size_t)b * L;  // first drafter row of this request
  // Tables of the row stage [BDDT §3, §4.3]: candidate words (staged with
  // the key in the lp slot and the id word in the tok slot), row maxima and
  // the fixed-point partial sums of every row.
  if (wid == 0) {
    // lane d < L: row d's maximum and the log of its normaliser, the sum of
    // its S <= 32 fixed-point partial sums (all requested at once)
    const float m = lane < L ? a.row_max[r0 + lane] : -INFINITY;
    uint64_t part[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) part[j] = (lane < L && j < S) ? a.row_sum[(r0 + lane) * S + j] : 0ull;
    uint64_t sum = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) sum += part[j];
    if (lane < L) {
      sh.rmax[lane] = m;
      sh.rlse[lane] = m == -INFINITY ? INFINITY : lse_from_fixed(sum);
    }
  } else {
    for (int i = tid - 64; i < LK; i += kBlock - 64) {
      const uint64_t wd = a.row_cand[r0 * K + i];
      sh.tok[i] = (int32_t)(uint32_t)wd;
      sh.lp[i] = __uint_as_float((uint32_t)(wd >> 32));
    }
    if (wid == 1 && a.status) {  // L <= 64 row flags, one per lane, OR-reduced
      const uint32_t f = wave_or_dpp(lane < L ? (uint32_t)a.row_flags[r0 + lane] : 0u);
      if (lane == 0) a.status[b] = (int32_t)f;
    }
  }
  __syncthreads();
  // log-probabilities: lp = (x - m) - lse, or at temperature 0 the argmax
  // limit (0 - lse for the maximum, -inf elsewhere)
  for (int i = tid; i < LK; i += kBlock) {
    const int row = i / K;
    const float x = order_to_float(__float_as_uint(sh.lp[i]));
    const int id = (int)(0xFFFFFFFFu - (uint32_t)sh.tok[i]);
    const float m = sh.rmax[row];
    float lp = -INFINITY;
    if (m != -INFINITY) {
      const float d = (a.mode == 2) ? ((x == m) ? 0.0f : -INFINITY) : (x - m);
      lp = d - sh.rlse[row];
    }
    sh.tok[i] = id;
    sh.lp[i] = lp;
    if (a.topk_tok) a.topk_tok[r0 * K + i] = id;
    if (a.topk_lp) a.topk_lp[r0 * K + i] = lp;
  }
  __syncthreads();
  if (wid == 0) {
    const int nn = K > 1 ? tree_pops<true>(sh, a.L, K, a.N) : tree_pops<false>(sh, a.L, K, a.N);
    if (lane == 0) {
      sh.nn = nn;
      sh.cmd = 0;
    }
    __syncthreads();
  } else {
    for (;;) {
      __syncthreads();
      if (sh.cmd == 0) break;
      sort_over(sh, sh.nover);
    }
  }
  __syncthreads();
  const int nn = sh.nn;
  const int T = a.N + 1;
  for (int i = tid; i < T; i += kBlock) {
    const size_t o = (size_t)b * T + i;
    int tk = -1, pa = -1, de = -1;
    float sc = -INFINITY;
    if (i == 0) {
      tk = a.root_tokens[b];
      de = 0;
      sc = 0.0f;
    } else if (i < nn) {
      const uint64_t k = sh.nkey[i];
      const uint32_t lo = (uint32_t)k;
      de = (int)(lo >> 25);
      pa = (int)((lo >> 14) & 0x7FFu);
      tk = sh.tok[(de - 1) * K + (int)((lo >> 9) & 31u)];
      sc = __uint_as_float((uint32_t)(k >> 32));
    }
    a.tokens[o] = tk;
    a.parents[o] = pa;
    a.depths[o] = de;
    a.scores[o] = sc;
    sh.par[i] = pa;
  }
  if (tid == 0) a.num_nodes[b] = nn;
  if (!a.mask) return;
  __syncthreads();
  // one thread per row: a single walk up the ancestor chain, whose node
  // indices decrease, emits the row's words from the highest to the lowest
  const int W = (T + 63) >> 6;
  for (int i = tid; i < T; i += kBlock) {
    uint64_t* out = a.mask + ((size_t)b * T + i) * W;
    int j = i < nn ? i : -1;
    for (int w = W - 1; w >= 0; --w) {
      uint64_t bits = 0;
      while (j >= 64 * w) {
        bits |= 1ull << (j - 64 * w);
        j = sh.par[j];
      }
      out[w] = bits;
    }
  }
}

}  // namespace

hipError_t launch_tree(const TreeArgs& t, int batch, hipStream_t st) {
  hipLaunchKernelGGL(k_tree, dim3(batch), dim3(kBlock), 0, st, t);
  return hipGetLastError();
}

}  // namespace ddt
