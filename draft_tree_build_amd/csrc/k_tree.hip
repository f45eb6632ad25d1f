// Draft-tree log-probabilities, best-first tree and ancestor bitmask on
// gfx950 (k_tree).
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, cited as [BDDT <section>].
//
// One workgroup per request, two kernels for the same tree: k_tree (below,
// node budgets up to 128) runs the pops of the best-first search; k_tree_level
// (further down, larger budgets) selects the same prefixes level by level.
// Both first turn the row stage's candidate words, maxima and fixed-point
// sums into the top-K tables (token, log-probability) per position.
//
// k_tree: wave 0 runs the N pops of the best-first search [BDDT §4.3, App. A]. The best pending candidates are kept sorted
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

// The top-K tables of one request from the row stage [BDDT §3, §4.3]:
// candidate words (staged with the key in the lp slot and the id word in the
// tok slot), row maxima and the fixed-point partial sums of every row give
// tok[d][k] and lp[d][k] = (x - m) - lse (at temperature 0 the argmax limit:
// 0 - lse for the maximum, -inf elsewhere). Sixteen threads share a row's
// S <= 32 partial sums (two each, summed over the sixteen lanes), and the
// first of them takes lse.
template <int BLOCK>
__device__ void build_tables(const TreeArgs& a, int b, int32_t* tok, float* lp, float* rmax,
                             float* rlse) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = a.K, L = a.L, S = a.S;
  const int LK = L * K;
  const size_t r0 = (size_t)b * L;  // first drafter row of this request
  for (int t = tid; t < 64 * 16; t += BLOCK) {
    const int row = t >> 4, sub = t & 15;
    uint64_t sum = 0;
    float m = -INFINITY;
    if (row < L) {
      const uint64_t* ps = a.row_sum + (r0 + row) * S;
      const uint64_t p0 = sub < S ? ps[sub] : 0ull;
      const uint64_t p1 = sub + 16 < S ? ps[sub + 16] : 0ull;
      if (sub == 0) m = a.row_max[r0 + row];
      sum = p0 + p1;
    }
    // the sum over the row's sixteen lanes, by DPP: lane ^ 1, lane ^ 2,
    // the other quad of each 8, the other 8 of each 16
    sum += dpp_src64<0xB1, 0xF>(0ull, sum);
    sum += dpp_src64<0x4E, 0xF>(0ull, sum);
    sum += dpp_src64<0x141, 0xF>(0ull, sum);
    sum += dpp_src64<0x140, 0xF>(0ull, sum);
    if (row < L && sub == 0) {
      rmax[row] = m;
      rlse[row] = m == -INFINITY ? INFINITY : lse_from_fixed(sum);
    }
  }
  for (int i = tid; i < LK; i += BLOCK) {
    const uint64_t wd = a.row_cand[r0 * K + i];
    tok[i] = (int32_t)(uint32_t)wd;
    lp[i] = __uint_as_float((uint32_t)(wd >> 32));
  }
  if (wid == 0 && a.status) {  // L <= 64 row flags, one per lane, OR-reduced
    const uint32_t f = wave_or_dpp(lane < L ? (uint32_t)a.row_flags[r0 + lane] : 0u);
    if (lane == 0) a.status[b] = (int32_t)f;
  }
  __syncthreads();
  for (int i = tid; i < LK; i += BLOCK) {
    const int row = i / K;
    const float x = order_to_float(__float_as_uint(lp[i]));
    const int id = (int)(0xFFFFFFFFu - (uint32_t)tok[i]);
    const float m = rmax[row];
    float l = -INFINITY;
    if (m != -INFINITY) {
      const float d = (a.mode == 2) ? ((x == m) ? 0.0f : -INFINITY) : (x - m);
      l = d - rlse[row];
    }
    tok[i] = id;
    lp[i] = l;
    if (a.topk_tok) a.topk_tok[r0 * K + i] = id;
    if (a.topk_lp) a.topk_lp[r0 * K + i] = l;
  }
  __syncthreads();
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
  build_tables<kBlock>(a, b, sh.tok, sh.lp, sh.rmax, sh.rlse);
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

// ======================================================================
// Level-synchronous selection (k_tree_level) [BDDT §4.2, §4.3, App. A].
//
// The best-first search returns the N best prefixes of the restricted set
// under the total order (score desc, depth asc, within-depth position asc),
// where the within-depth position orders the prefixes of one depth by
// (score desc, parent's position asc, rank asc). The tree is therefore the
// set of prefixes whose score beats the N-th best score theta*, plus the
// first N - F prefixes tied at theta* (F = the number strictly above it)
// in (depth, within-depth position) order, numbered in that total order.
// The whole workgroup computes it in three phases:
//
//  1. Depth by depth, the children of the kept nodes of the previous depth
//     whose score is above a running threshold th are stored (a parent's
//     qualifying children are a run of its first ranks: log-probabilities
//     are sorted). th starts at -inf; whenever N or more nodes are stored,
//     th becomes the N-th best stored score (a radix select on the score
//     bits; any N prefixes at or above a score make it a lower bound of
//     theta*) and the nodes not above it are dropped. Nothing below th can
//     be in the tree (a descendant never beats its ancestor), so the stored
//     set ends as exactly the F < N prefixes above theta* = th.
//  2. The stored nodes are ordered: per depth by (score, parent's
//     within-depth rank, rank) -- rank counting, depth after depth -- then
//     across depths by (score, depth, within-depth rank): each node counts
//     the nodes of the other depths ahead of it by binary searches in their
//     sorted score lists. Node i of the tree is the i-th in this order.
//  3. The prefixes tied at th follow, depth by depth: at each depth the
//     parents in within-depth order (stored nodes, then the tied nodes taken
//     at the depth before) with, per parent, the run of ranks whose score
//     equals th, until N nodes are placed (or the restricted set runs out);
//     depths without such a run take no round.
//
// Scores are sums of log-probabilities: <= 0 and never -0, so their raw
// bits order them in reverse (the select and the per-depth keys use them).

constexpr int kLB = 1024;           // threads of k_tree_level
constexpr int kLW = kLB / 64;      // its waves
constexpr int kCap = 8192;         // stored nodes (above the running threshold)
constexpr int kPPT = kCap / kLB;   // parents per thread when a depth's parents fill the store
constexpr int kMaxN = 1024;
constexpr uint16_t kRootRef = 0xFFFFu;


struct LevelShared {
  int32_t tok[kMaxLK];             // top-K tokens, [L, K]
  float lp[kMaxLK];                // their log-probabilities
  float rmax[64];
  float rlse[64];
  float s_score[kCap];             // stored nodes: score,
  uint16_t s_par[kCap];            //   parent (stored index, kRootRef at depth 1),
  uint8_t s_depth[kCap];           //   depth and rank
  uint8_t s_rank[kCap];
  int32_t s_tmp[kCap];             // counts and scans; phase 2 buckets; phase 3 scans
  int32_t hist[256];
  int32_t red[kLW];
  uint32_t red2[2 * kLW];
  int32_t dbeg[64 + 2];            // first stored index of each depth
  int32_t dtot[64 + 2];            // phase 3: tied children per depth
  uint32_t o_bits[kMaxN];          // stored nodes of each depth in within-depth
  uint16_t o_fi[kMaxN];            //   order: score bits, node index and
  uint16_t o_u[kMaxN];             //   stored index
  uint64_t keytmp[kMaxN];          // phase 2: within-depth keys
  uint8_t tlo[kMaxN];              // phase 3, per stored node: first rank and
  uint8_t tcnt[kMaxN];             //   count of its children scored th
  uint16_t n_par[kMaxT];           // the tree, by node index
  uint8_t n_depth[kMaxT];
  uint8_t n_rank[kMaxT];
  float n_score[kMaxT];
  int32_t bc[4];                   // values broadcast to the workgroup
};

// Inclusive prefix sum over the 64 lanes by DPP (no LDS round trip): within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes without a source
// add 0), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Exclusive prefix sum of arr[0..n) in place (n <= kCap, kScanPer
// consecutive entries per thread); returns the total. The caller has a
// barrier between the writes of arr and the call.
constexpr int kScanPer = kCap / kLB;
__device__ int level_scan(int32_t* arr, int n, int32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int per = (n + kLB - 1) / kLB;   // consecutive entries per thread (<= kScanPer)
  const int i0 = per * tid;
  int v[kScanPer];
  int s = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = 0;
    if (j >= per) break;
    v[j] = i0 + j < n ? arr[i0 + j] : 0;
    s += v[j];
  }
  const int inc = wave_scan_dpp(s);
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kLW; ++w) {
    const int t = red[w];
    before += w < wid ? t : 0;
    total += t;
  }
  int run = before + inc - s;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (j >= per) break;
    if (i0 + j < n) arr[i0 + j] = run;
    run += v[j];
  }
  __syncthreads();
  return total;
}

// Ranks r of the row l[0..K) (non-increasing) with fl(ps + l[r]) > th
// (STRICT) or >= th: the sums are non-increasing in r, so a binary search.
template <bool STRICT>
__device__ __forceinline__ int count_ranks(float ps, const float* l, int K, float th) {
  int lo = 0, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const float s = ps + l[mid];
    if (STRICT ? (s > th) : (s >= th)) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// The rank-th smallest (1-based) of the score bits of s_score[0..n): a
// radix select, eight bits per pass, counting in an LDS histogram. The bits
// all keys share (their AND equals their OR there) are skipped: the passes
// start at the highest bit in which the keys differ.
__device__ uint32_t select_bits(LevelShared& sh, int n, int rank) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
  // (each thread's keys are requested together, then combined: an LDS
  // round trip per batch, not per key; likewise below)
  for (int i0 = tid; i0 < n; i0 += 4 * kLB) {
    uint32_t x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = __float_as_uint(sh.s_score[min(i0 + u * kLB, n - 1)]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kand &= x[u];
      kor |= x[u];
    }
  }
  kand = dpp_reduce(kand, 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return x & y; });
  kor = wave_or_dpp(kor);
  if (lane == 0) {
    sh.red2[2 * wid] = kand;
    sh.red2[2 * wid + 1] = kor;
  }
  __syncthreads();
  kand = 0xFFFFFFFFu;
  kor = 0u;
#pragma unroll
  for (int w = 0; w < kLW; ++w) {
    kand &= sh.red2[2 * w];
    kor |= sh.red2[2 * w + 1];
  }
  const uint32_t diff = kand ^ kor;               // bits in which the keys differ
  if (diff == 0u) return kand;                     // all keys equal
  const int top = 31 - __builtin_clz(diff);        // highest differing bit
  uint32_t prefix = kand & ~((2u << top) - 1u);    // the shared high bits
  int need = rank;
  for (int shift = top - 7; shift > -8; shift -= 8) {
    const int sh_lo = max(shift, 0);
    const int nb = shift >= 0 ? 8 : 8 + shift;     // bits in this pass
    // (the previous pass's histogram readers passed the barrier before bc)
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    const uint32_t hmask = sh_lo + nb >= 32 ? 0u : ~((1u << (sh_lo + nb)) - 1u);
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i0 = tid; i0 < n; i0 += 4 * kLB) {
      uint32_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = __float_as_uint(sh.s_score[min(i0 + u * kLB, n - 1)]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * kLB < n && (x[u] & hmask) == prefix) atomicAdd(&sh.hist[(x[u] >> sh_lo) & dmask], 1);
    }
    __syncthreads();
    if (wid == 0) {
      const int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
      const int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      const int sum = h0 + h1 + h2 + h3;
      const int inc = wave_scan_dpp(sum);
      const int ex = inc - sum;
      if (ex < need && need <= inc) {
        int c = ex, bin = 4 * lane;
        if (c + h0 < need) {
          c += h0;
          ++bin;
          if (c + h1 < need) {
            c += h1;
            ++bin;
            if (c + h2 < need) {
              c += h2;
              ++bin;
            }
          }
        }
        sh.bc[0] = bin;
        sh.bc[1] = c;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bc[0] << sh_lo;
    need -= sh.bc[1];
  }
  return prefix;
}

// Number of entries of the non-decreasing arr[0..n) that are < x (LE:
// <= x).
template <bool LE>
__device__ __forceinline__ int count_below(const uint32_t* arr, int n, uint32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (LE ? (arr[mid] <= x) : (arr[mid] < x)) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kLB) void k_tree_level(TreeArgs a) {
  __shared__ LevelShared sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = a.K, L = a.L, N = a.N;
  build_tables<kLB>(a, b, sh.tok, sh.lp, sh.rmax, sh.rlse);

  // ---- phase 1: the nodes above the running threshold, depth by depth
  const int kshift = K <= 1 ? 0 : 32 - __builtin_clz((unsigned)(K - 1));  // ranks per grid row: 2^kshift >= K
  const int kmask = (1 << kshift) - 1;
  float th = -INFINITY;
  int nS = 0;
  int prev_b = 0, prev_e = 0;   // stored range of the previous depth
  int D = 0;                    // deepest depth with stored nodes
  for (int d = 1; d <= L; ++d) {
    const float* lrow = sh.lp + (d - 1) * K;
    int nparents = d == 1 ? 1 : prev_e - prev_b;
    if (nparents == 0) break;
    int lev_b = nS;
    if (tid == 0) sh.dbeg[d] = nS;
    int cur = 0;                // parents done, counted from prev_b

    // th <- the N-th best stored score; keep the nodes above it (stable,
    // parent links and range bounds renumbered)
    auto select_compact = [&]() __attribute__((always_inline)) {
      const uint32_t tb = select_bits(sh, nS, N);
      th = __uint_as_float(tb);
      for (int i0 = tid; i0 < nS; i0 += 4 * kLB) {
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = __float_as_uint(sh.s_score[min(i0 + u * kLB, nS - 1)]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i0 + u * kLB < nS) sh.s_tmp[i0 + u * kLB] = x[u] < tb ? 1 : 0;
      }
      __syncthreads();
      const int kept = level_scan(sh.s_tmp, nS, sh.red);
      // new index of stored index x: the survivors before it
      auto renum = [&](int x) { return x < nS ? sh.s_tmp[x] : kept; };
      float rs[kPPT];
      uint32_t rw[kPPT];        // parent (16 bits) | depth (8) | rank (8); ~0: dropped
#pragma unroll
      for (int k = 0; k < kPPT; ++k) rw[k] = ~0u;
#pragma unroll
      for (int k = 0; k < kPPT; ++k) {
        const int i = tid + k * kLB;
        if (i >= nS) break;
        if (__float_as_uint(sh.s_score[i]) < tb) {
          rs[k] = sh.s_score[i];
          const uint16_t pr = sh.s_par[i];
          const uint32_t np_ = pr == kRootRef ? kRootRef : (uint32_t)sh.s_tmp[pr];
          rw[k] = (np_ << 16) | ((uint32_t)sh.s_depth[i] << 8) | sh.s_rank[i];
        }
      }
      const int nb = renum(prev_b), ncur = renum(prev_b + cur), ne = renum(prev_e);
      const int nlev = renum(lev_b);
      int ndb = 0;
      if (tid < d) ndb = renum(sh.dbeg[tid + 1]);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPPT; ++k) {
        if (tid + k * kLB >= nS) break;
        if (rw[k] != ~0u) {     // its new index: s_tmp is not written here
          const int dst = sh.s_tmp[tid + k * kLB];
          sh.s_score[dst] = rs[k];
          sh.s_par[dst] = (uint16_t)(rw[k] >> 16);
          sh.s_depth[dst] = (uint8_t)(rw[k] >> 8);
          sh.s_rank[dst] = (uint8_t)rw[k];
        }
      }
      if (tid < d) sh.dbeg[tid + 1] = ndb;
      if (d > 1) {
        prev_b = nb;
        prev_e = ne;
        cur = ncur - nb;
        nparents = ne - nb;
      }
      lev_b = nlev;
      nS = kept;
      __syncthreads();
    };

    // One pass when every qualifying child fits in the store: the parents'
    // runs (binary searches in the sorted row), their offsets (a scan), and
    // the children written on a (parent, rank) grid, one child per thread.
    bool full = false;
    if (nparents <= 64) {
      // Few parents: wave 0 alone counts their runs, scans them by DPP and
      // writes the children (a lane per parent, its run in rank order), and
      // one barrier publishes them; the same positions as the grid below.
      if (tid < 64) {
        const float ps = d == 1 ? 0.0f : (tid < nparents ? sh.s_score[prev_b + tid] : 0.0f);
        const int c = tid < nparents ? count_ranks<true>(ps, lrow, K, th) : 0;
        const int incl = wave_scan_dpp(c);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (total <= kCap - nS) {
          const int q0 = nS + incl - c;
          for (int r = 0; r < c; ++r) {
            sh.s_score[q0 + r] = ps + lrow[r];
            sh.s_par[q0 + r] = d == 1 ? kRootRef : (uint16_t)(prev_b + tid);
            sh.s_depth[q0 + r] = (uint8_t)d;
            sh.s_rank[q0 + r] = (uint8_t)r;
          }
        }
        if (tid == 0) sh.bc[3] = total;
      }
      __syncthreads();
      const int total = sh.bc[3];
      if (total <= kCap - nS) {
        nS += total;
        cur = nparents;
        full = nS >= N;
      }
    } else {
      for (int j = tid; j < nparents; j += kLB)
        sh.s_tmp[j] = count_ranks<true>(d == 1 ? 0.0f : sh.s_score[prev_b + j], lrow, K, th);
      __syncthreads();
      const int total = level_scan(sh.s_tmp, nparents, sh.red);
      if (total <= kCap - nS) {
        const int cells = nparents << kshift;
        for (int t0 = 0; t0 < cells; t0 += 4 * kLB) {
          // four grid cells per thread: every load first, then the stores
          int off[4], c[4];
          float ps[4], l[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = min(t0 + u * kLB + tid, cells - 1);
            const int j = t >> kshift, r = t & kmask;
            off[u] = sh.s_tmp[j];
            c[u] = j + 1 < nparents ? sh.s_tmp[j + 1] : total;
            ps[u] = d == 1 ? 0.0f : sh.s_score[prev_b + j];
            l[u] = lrow[min(r, K - 1)];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = t0 + u * kLB + tid;
            const int j = t >> kshift, r = t & kmask;
            if (t < cells && r < c[u] - off[u]) {
              const int q = nS + off[u] + r;
              sh.s_score[q] = ps[u] + l[u];
              sh.s_par[q] = d == 1 ? kRootRef : (uint16_t)(prev_b + j);
              sh.s_depth[q] = (uint8_t)d;
              sh.s_rank[q] = (uint8_t)r;
            }
          }
        }
        nS += total;
        cur = nparents;
        full = nS >= N;
        __syncthreads();
      }
    }
    if (full) select_compact();
    // Otherwise in chunks of parents whose runs fit, the threshold rising
    // between chunks.
    while (cur < nparents) {
      const int rem = nparents - cur;
      for (int j = tid; j < rem; j += kLB) {
        const float ps = d == 1 ? 0.0f : sh.s_score[prev_b + cur + j];
        sh.s_tmp[j] = count_ranks<true>(ps, lrow, K, th);
      }
      __syncthreads();
      const int total = level_scan(sh.s_tmp, rem, sh.red);
      const int room = kCap - nS;
      int take = rem;
      if (total > room) {       // the parents whose runs all fit
        if (tid == 0) sh.bc[2] = rem;
        __syncthreads();
        for (int j = tid; j < rem; j += kLB) {
          const int end = j + 1 < rem ? sh.s_tmp[j + 1] : total;
          if (end > room) atomicMin(&sh.bc[2], j);
        }
        __syncthreads();
        take = sh.bc[2];
      }
      const int added = take < rem ? sh.s_tmp[take] : total;
      for (int j = tid; j < take; j += kLB) {
        const int off = sh.s_tmp[j];
        const int c = (j + 1 < rem ? sh.s_tmp[j + 1] : total) - off;
        const int p = prev_b + cur + j;
        const float ps = d == 1 ? 0.0f : sh.s_score[p];
        for (int r = 0; r < c; ++r) {
          const int q = nS + off + r;
          sh.s_score[q] = ps + lrow[r];
          sh.s_par[q] = d == 1 ? kRootRef : (uint16_t)p;
          sh.s_depth[q] = (uint8_t)d;
          sh.s_rank[q] = (uint8_t)r;
        }
      }
      nS += added;
      cur += take;
      __syncthreads();
      if (nS >= N) select_compact();
    }
    prev_b = lev_b;
    prev_e = nS;
    if (prev_e == prev_b) break;  // no node above th at depth d: none deeper
    D = d;
  }
  const int F = nS;
  if (tid == 0) sh.dbeg[D + 1] = F;
  __syncthreads();

  // ---- phase 2: order the stored nodes, depth by depth by (score, parent's
  // within-depth rank, rank), then across depths. The stored depth-1 nodes
  // are the root's ranks 0, 1, ... in order, so their within-depth rank is
  // their rank; each deeper depth is ranked by counting, and its scatter
  // into the sorted lists shares a pass with the next depth's keys.
  int need = N - F, taken = 0;
  for (int d = 1; d <= D + 1; ++d) {
    // scatter of depth d - 1 (its ranks are final), keys of depth d
    if (d >= 2) {
      const int pb = sh.dbeg[d - 1], pm = sh.dbeg[d] - pb;
      for (int i = tid; i < pm; i += kLB) {
        const int u = pb + i;
        const int rho = d == 2 ? i : sh.s_tmp[u];
        if (d == 2) sh.s_tmp[u] = i;
        sh.o_bits[pb + rho] = __float_as_uint(sh.s_score[u]);
        sh.o_u[pb + rho] = (uint16_t)u;
      }
    }
    if (d > D || d == 1) {
      __syncthreads();
      continue;
    }
    const int db = sh.dbeg[d], m = sh.dbeg[d + 1] - db;
    // keys (the parents' ranks, depth d - 1: the rank itself at depth 1)
    // and the depth's own rank counters cleared (disjoint entries)
    for (int i = tid; i < m; i += kLB) {
      const int u = db + i;
      const int pr = sh.s_par[u];
      const uint32_t prho = d == 2 ? (uint32_t)sh.s_rank[pr] : (uint32_t)sh.s_tmp[pr];
      sh.keytmp[i] = ((uint64_t)__float_as_uint(sh.s_score[u]) << 32) | (prho << 5) | sh.s_rank[u];
      sh.s_tmp[u] = 0;
    }
    __syncthreads();
    // rank counting: node u compares with a slice of the depth's nodes,
    // eight keys requested per round trip
    const int parts = m > 0 ? max(1, min(kLB / m, 64)) : 1;
    const int per = (m + parts - 1) / parts;
    for (int t = tid; t < m * parts; t += kLB) {
      const int u = t % m, part = t / m;
      const uint64_t ku = sh.keytmp[u];
      const int v0 = part * per, v1 = min(m, v0 + per);
      int c = 0;
      for (int v = v0; v < v1; v += 8) {
        uint64_t kv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = sh.keytmp[min(v + j, v1 - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) c += (v + j < v1 && kv[j] < ku) ? 1 : 0;
      }
      if (c) atomicAdd(&sh.s_tmp[db + u], c);
    }
    __syncthreads();
  }
  // position in the tree: the within-depth rank plus the nodes of other
  // depths ahead (shallower ones at equal score come first); and, for the
  // ties at th, each node's run of children scored exactly th (ranks
  // [tlo, tlo + tcnt)) with the per-depth totals
  for (int i = tid; i <= 64 + 1; i += kLB) sh.dtot[i] = 0;
  __syncthreads();
  for (int u = tid; u < F; u += kLB) {
    const int d = sh.s_depth[u];
    const uint32_t x = __float_as_uint(sh.s_score[u]);
    const int rho = d == 1 ? u - sh.dbeg[1] : sh.s_tmp[u];
    int pos = rho;
    for (int e = 1; e <= D; ++e) {
      if (e == d) continue;
      const int eb = sh.dbeg[e], en = sh.dbeg[e + 1] - eb;
      pos += e < d ? count_below<true>(sh.o_bits + eb, en, x) : count_below<false>(sh.o_bits + eb, en, x);
    }
    sh.o_fi[sh.dbeg[d] + rho] = (uint16_t)(1 + pos);
    if (need > 0) {
      int lo = 0, hi = 0;
      if (d < L) {
        const float* lr = sh.lp + d * K;
        lo = count_ranks<true>(sh.s_score[u], lr, K, th);
        hi = count_ranks<false>(sh.s_score[u], lr, K, th);
      }
      sh.tlo[u] = (uint8_t)lo;
      sh.tcnt[u] = (uint8_t)(hi - lo);
      if (hi > lo) atomicAdd(&sh.dtot[d + 1], hi - lo);
    }
  }
  __syncthreads();
  for (int u = tid; u < F; u += kLB) {
    const int d = sh.s_depth[u];
    const int rho = d == 1 ? u - sh.dbeg[1] : sh.s_tmp[u];
    const int fi = sh.o_fi[sh.dbeg[d] + rho];
    const uint16_t pr = sh.s_par[u];
    sh.n_par[fi] = pr == kRootRef ? 0 : sh.o_fi[sh.dbeg[d - 1] + (d == 2 ? pr - sh.dbeg[1] : sh.s_tmp[pr])];
    sh.n_depth[fi] = (uint8_t)d;
    sh.n_rank[fi] = sh.s_rank[u];
    sh.n_score[fi] = sh.s_score[u];
  }
  __syncthreads();

  // ---- phase 3: the prefixes tied at th, in (depth, within-depth) order;
  // depths without tied children (and no tied parents) take no round.
  int tb = 0, te = 0;           // tied nodes of the previous depth: F + 1 + [tb, te)
  int32_t* pscan = sh.s_tmp;    // per-parent counts, then offsets
  for (int d = 1; d <= L && need > 0; ++d) {
    const float* lrow = sh.lp + (d - 1) * K;
    // tied parents have tied children only where th + lp == th
    const int tlo_t = count_ranks<true>(th, lrow, K, th);
    const int tct = te > tb ? count_ranks<false>(th, lrow, K, th) - tlo_t : 0;
    const int rlo = d == 1 ? count_ranks<true>(0.0f, lrow, K, th) : 0;
    const int from_s = d == 1 ? count_ranks<false>(0.0f, lrow, K, th) - rlo : sh.dtot[d];
    if (from_s == 0 && tct == 0) {
      if (d > D) break;         // no stored node at depth d or deeper, no tied parent
      tb = te = taken;
      continue;
    }
    int take = 0;
    if (d == 1) {               // the root's run
      take = min(from_s, need);
      for (int j = tid; j < take; j += kLB) {
        const int fi = F + 1 + j;
        sh.n_par[fi] = 0;
        sh.n_depth[fi] = 1;
        sh.n_rank[fi] = (uint8_t)(rlo + j);
        sh.n_score[fi] = th;
      }
    } else {
      // parents in within-depth order: the stored nodes of depth d - 1,
      // then the tied nodes of depth d - 1
      const int ms = d - 1 <= D ? sh.dbeg[d] - sh.dbeg[d - 1] : 0;
      const int mb = d - 1 <= D ? sh.dbeg[d - 1] : 0;
      const int np = ms + (te - tb);
      for (int q = tid; q < np; q += kLB) pscan[q] = q < ms ? sh.tcnt[sh.o_u[mb + q]] : tct;
      __syncthreads();
      const int total = level_scan(pscan, np, sh.red);
      take = min(total, need);
      for (int q = tid; q < np; q += kLB) {
        const int off = pscan[q];
        if (off >= take) continue;
        const int c = min((q + 1 < np ? pscan[q + 1] : total) - off, take - off);
        int pfi, lo;
        if (q < ms) {
          pfi = sh.o_fi[mb + q];
          lo = sh.tlo[sh.o_u[mb + q]];
        } else {
          pfi = F + 1 + tb + (q - ms);
          lo = tlo_t;
        }
        for (int j = 0; j < c; ++j) {
          const int fi = F + 1 + taken + off + j;
          sh.n_par[fi] = (uint16_t)pfi;
          sh.n_depth[fi] = (uint8_t)d;
          sh.n_rank[fi] = (uint8_t)(lo + j);
          sh.n_score[fi] = th;
        }
      }
    }
    __syncthreads();
    tb = taken;
    te = taken + take;
    taken += take;
    need -= take;
  }
  const int nn = 1 + F + taken;

  // ---- the tree arrays and the mask rows
  const int T = N + 1;
  for (int i = tid; i < T; i += kLB) {
    const size_t o = (size_t)b * T + i;
    int tk = -1, pa = -1, de = -1;
    float sc = -INFINITY;
    if (i == 0) {
      tk = a.root_tokens[b];
      de = 0;
      sc = 0.0f;
    } else if (i < nn) {
      de = sh.n_depth[i];
      pa = sh.n_par[i];
      tk = sh.tok[(de - 1) * K + sh.n_rank[i]];
      sc = sh.n_score[i];
    }
    a.tokens[o] = tk;
    a.parents[o] = pa;
    a.depths[o] = de;
    a.scores[o] = sc;
  }
  if (tid == 0) a.num_nodes[b] = nn;
  if (!a.mask) return;
  // one thread per row: a single walk up the ancestor chain, whose node
  // indices decrease, emits the row's words from the highest to the lowest
  const int W = (T + 63) >> 6;
  for (int i = tid; i < T; i += kLB) {
    uint64_t* out = a.mask + ((size_t)b * T + i) * W;
    int j = i < nn ? i : -1;
    for (int w = W - 1; w >= 0; --w) {
      uint64_t bits = 0;
      while (j >= 64 * w) {
        bits |= 1ull << (j - 64 * w);
        j = j == 0 ? -1 : (int)sh.n_par[j];
      }
      out[w] = bits;
    }
  }
}

}  // namespace

// Both kernels build the same tree. The pops of k_tree cost ~0.2-0.3 us
// each; k_tree_level costs a roughly fixed number of workgroup-wide steps
// (~25-45 us per request whatever N). Measured (build stage, L = 16,
// V = 32,000 / 151,936): the pops win at N = 64 (35.4 / 43.6 against
// 35.9 / 45.4 us), the level selection from N = 80 (39.7 / 45.6 against
// 41.5 / 49.0 us; 46 against 165 us at N = 512). In argmax mode (draft
// temperature 0) the level selection walks every depth with a few parents
// each, at a near-fixed ~69 us, while the pops cost ~0.3 us each: 58
// against 69 us at N = 128, equal at N = 160, 79 against 70 us at N = 192
// (V = 151,936, K = 16).
constexpr int kLevelMinN = 72;
constexpr int kLevelMinNArgmax = 160;

hipError_t launch_tree(const TreeArgs& t, int batch, hipStream_t st) {
  const int min_n = t.mode == 2 ? kLevelMinNArgmax : kLevelMinN;
  if (t.N >= min_n) hipLaunchKernelGGL(k_tree_level, dim3(batch), dim3(kLB), 0, st, t);
  else hipLaunchKernelGGL(k_tree, dim3(batch), dim3(kBlock), 0, st, t);
  return hipGetLastError();
}

}  // namespace ddt
