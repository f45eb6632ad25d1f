// Tree-attention verify on gfx950.
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, cited as [BDDT <section>]: the tree is
// verified in one target forward with an ancestor-only mask (Abstract,
// §4.1); the pages' implementation used a dense-mask SDPA call (App. B).
// Here every tree query attends to the whole prefix and to the tree keys
// selected by its 64-bit mask words; the prefix part is a dense contraction
// and runs on MFMA.
//
// bf16, D = 128 (k_attn_mfma): one workgroup = 4 waves = 128 query rows of
// one (request, kv-head) -- rows are node-major, the g = Hq/Hkv query heads
// of a node adjacent, so GQA shares every K/V tile across g heads. Key tiles
// of 64 rows are staged through LDS (K row-major, V transposed, both XOR
// swizzled). Per wave and tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16
// (lane = query row), online softmax in fp32 (exp2 domain), O^T += V^T P^T
// with P split into two bf16 parts (hi + lo) so the weights stay ~fp32 exact.
// The key tile list is prefix tiles then tree tiles (mask applied); long
// lists are split across workgroups and merged by a second kernel
// (log-sum-exp weights).
//
// f32 (k_attn_simple): one thread per query row, fp32 throughout.
#include "ddtree_device.h"
#include "ddtree_internal.h"

#include <algorithm>

namespace ddt {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerWave = 32;
constexpr int kWavesA = 4;
constexpr int kTileRows = kRowsPerWave * kWavesA;  // 128
constexpr int kKeys = 64;
constexpr float kLog2e = 1.4426950408889634f;

// K tile: 64 rows of 256 bytes (128 dims), row r at byte r*272 + (r/8)*64.
// The padding puts the 8 lanes of a 128-bit fragment read -- keys
// {0..3, 8..11} + c or {4..7, 12..15} + c -- on 8 distinct 16-byte bank
// groups, and every fragment offset of a lane is a compile-time immediate.
constexpr int kKRow = kD * 2 + 16;
constexpr int kKBytes = (kKeys - 1) * kKRow + (kKeys / 8 - 1) * 64 + kD * 2;
__device__ __forceinline__ int k_row_off(int key) { return key * kKRow + (key >> 3) * 64; }
// V^T tile: [128 dims][8 chunks of 8 keys] = 128 bytes per dim, chunk index
// XOR-swizzled by sw(dim) = (dim ^ (dim >> 3)) & 7. Fragment reads (32
// consecutive dims) and transposed writes (dims 8 apart) both spread over
// the banks; for dim = 32 db + n, sw = ((n ^ (n >> 3)) & 7) ^ 4 (db & 1).
constexpr int kVBytes = kKeys * kD * 2;
__device__ __forceinline__ int v_lds_off(int dim, int chunk) {
  int sw = (dim ^ (dim >> 3)) & 7;
  return dim * (kKeys * 2) + ((chunk ^ sw) << 4);
}

struct AttnSplit {
  int nsplit;
  int row_tiles;
  int total;    // work items: batch * Hkv * nsplit * row_tiles
  int per_xcd;  // work items per XCD slice of the grid
};

constexpr int kXcds = 8;

// One workgroup = 128 query rows of one (request, kv-head) over one range of
// key tiles. Grid: 1-D, XCD-aware -- consecutive workgroup ids go to
// different XCDs, so work item w runs as workgroup (w % per_xcd) * 8 + w /
// per_xcd, which keeps all row tiles of one (request, kv-head, split) on one
// XCD and its K/V tiles in that XCD's L2. Key tiles are double-buffered in
// LDS: tile t+1 is fetched into registers while tile t is computed.
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a, AttnSplit pl, float* part_o,
                                                      float* part_ml) {
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][kKBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2][kVBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = (int)(blockIdx.x % kXcds) * pl.per_xcd + (int)(blockIdx.x / kXcds);
  if (wi >= pl.total) return;
  const int nsplit = pl.nsplit, row_tiles = pl.row_tiles;
  const int xt = wi % row_tiles;
  const int z = (wi / row_tiles) % nsplit;
  const int bhi = wi / (row_tiles * nsplit);
  const int b = bhi / a.Hkv, hk = bhi - (bhi / a.Hkv) * a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int T = a.T;
  const int R = T * g;
  const int nn = min(max(a.num_nodes[b], 0), T);
  const int nvalid_rows = nn * g;
  const int tile_row0 = xt * kTileRows;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v);
  uint16_t* O = static_cast<uint16_t*>(a.out);

  // rows of this lane: query row n = lane % 32 of wave w
  const int gq = lane >> 5;           // lane group (0/1)
  const int n = lane & 31;
  const int row = tile_row0 + w * kRowsPerWave + n;
  const int node = row / g;
  const int head = hk * g + (row - node * g);
  const bool row_valid = row < nvalid_rows;

  if (tile_row0 >= nvalid_rows) {
    // padding rows only: split 0 writes the zeros
    if (z == 0 && row < R) {
      uint16_t* o = O + (((size_t)b * T + node) * a.Hq + head) * kD;
      for (int c = gq; c < kD / 8; c += 2) reinterpret_cast<uint4*>(o)[c] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  // ---- key tiles of this row tile: prefix tiles then tree tiles
  const int P = max(a.prefix_lens[b], 0);
  const int np = (P + kKeys - 1) / kKeys;
  const int last_row = min(tile_row0 + kTileRows, nvalid_rows) - 1;
  const int max_node = last_row / g;  // ancestors have smaller indices
  const int nt = (max_node + 1 + kKeys - 1) / kKeys;
  const int ntiles = np + nt;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t_begin = min(z * per, ntiles), t_end = min(t_begin + per, ntiles);
  const size_t kv0 = (size_t)a.kv_offsets[b];
  const int W = (T + 63) >> 6;
  const float c_log2 = a.scale * kLog2e;

  // ---- Q fragments (B operand of S^T = K Q^T): dims 16 ks + 8 gq + 0..7
  bf16x8 qf[8];
  {
    const uint16_t* qp = Q + (((size_t)b * T + node) * a.Hq + head) * kD + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 u = row_valid ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  floatx16 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // staging of one K/V tile: lane covers dim chunk dc and keys
  // k0, k0+1, k0+8, k0+9 with k0 = 16 w + 2 kq
  const int dc = lane & 15, kq = lane >> 4;
  const int k0 = 16 * w + 2 * kq;
  uint4 sk[4], sv[4];
  auto tile_rows = [&](int t, int* base, int* nvalid) __attribute__((always_inline)) {
    if (t < np) {
      *base = t * kKeys;
      *nvalid = min(kKeys, P - t * kKeys);
    } else {
      const int tt = t - np;
      *base = P + tt * kKeys;
      *nvalid = min(kKeys, nn - tt * kKeys);
    }
  };
  // per-lane element offsets inside a tile (32-bit); the tile base is uniform
  const uint32_t row_elems = (uint32_t)a.Hkv * kD;
  const uint32_t lane_off0 = (uint32_t)k0 * row_elems + hk * kD + 8 * dc;
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    int base, nvalid;
    tile_rows(t, &base, &nvalid);
    const int64_t r0 = (int64_t)kv0 + base;  // first key row of the tile
    const int64_t lim = min((int64_t)nvalid, a.total_rows - r0);
    const size_t tb = (r0 < a.total_rows) ? (size_t)r0 * row_elems : 0;
    const uint16_t* kt = Kg + tb;
    const uint16_t* vt = Vg + tb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jk = (j & 1) + 8 * (j >> 1);
      const bool ok = (int64_t)(k0 + jk) < lim;
      // out-of-range keys read the tile's first row (or row 0) and are zeroed
      const uint32_t off = ok ? lane_off0 + (uint32_t)jk * row_elems : (uint32_t)(hk * kD + 8 * dc);
      const uint4 kx = *reinterpret_cast<const uint4*>(kt + off);
      const uint4 vx = *reinterpret_cast<const uint4*>(vt + off);
      sk[j] = ok ? kx : make_uint4(0, 0, 0, 0);
      sv[j] = ok ? vx : make_uint4(0, 0, 0, 0);
    }
  };
  // K: 128-bit writes; V: transposed 32-bit writes of key pairs
  auto write_tile = [&](int bf) __attribute__((always_inline)) {
    unsigned char* kl = k_lds[bf];
    unsigned char* vl = v_lds[bf];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + (j & 1) + 8 * (j >> 1);
      *reinterpret_cast<uint4*>(kl + k_row_off(key) + 16 * dc) = sk[j];
    }
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const uint4 va = sv[2 * hp], vb = sv[2 * hp + 1];
      const int key = k0 + 8 * hp;  // even; key+1 in the same 8-key chunk
      const uint32_t aw[4] = {va.x, va.y, va.z, va.w};
      const uint32_t bw[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (aw[e >> 1] >> 16) : (aw[e >> 1] & 0xFFFFu);
        const uint32_t hi = (e & 1) ? (bw[e >> 1] & 0xFFFF0000u) : (bw[e >> 1] << 16);
        const int dim = 8 * dc + e;
        *reinterpret_cast<uint32_t*>(vl + v_lds_off(dim, key >> 3) + (key & 7) * 2) = lo | hi;
      }
    }
  };

  // the key permutation of the S^T A operand: A row m -> key pi(m), chosen so
  // that lane group gq's score registers v = 0..7 hold keys 8 gq + v and
  // v = 8..15 hold keys 16 + 8 gq + (v - 8) of each 32-key block
  const int m_a = lane & 31;
  const int pi_m = 8 * ((m_a >> 2) & 1) + 16 * (m_a >> 4) + 4 * ((m_a >> 3) & 1) + (m_a & 3);
  const int kfrag0 = k_row_off(pi_m) + 16 * gq;  // + 32 ks, + kb block offset
  // V^T fragment addresses for dims 32 db + n: the 4 chunk offsets of this
  // lane; odd db flips swizzle bit 2, each db adds 32 dims * 128 bytes
  int vfrag[4];
  {
    const int sw = (n ^ (n >> 3)) & 7;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int chunk = 4 * (c >> 1) + 2 * (c & 1) + gq;  // kb = c/2, hf = c%2
      vfrag[c] = n * (kKeys * 2) + ((chunk ^ sw) << 4);
    }
  }

  // mask word of this lane's query row for tree tile t (prefetched with the tile)
  const uint64_t* mrow = a.mask + ((size_t)b * T + node) * W;
  auto load_mword = [&](int t) __attribute__((always_inline)) -> uint64_t {
    return (t >= np && row_valid) ? mrow[t - np] : 0ull;
  };
  int bf = 0;
  uint64_t mword_next = 0;
  if (t_begin < t_end) {
    load_tile(t_begin);
    mword_next = load_mword(t_begin);
    write_tile(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const bool has_next = t + 1 < t_end;
    const uint64_t mword = mword_next;
    if (has_next) {  // in flight while tile t is computed
      load_tile(t + 1);
      mword_next = load_mword(t + 1);
    }
    const unsigned char* kl = k_lds[bf];
    const unsigned char* vl = v_lds[bf];

    int base, nvalid;
    tile_rows(t, &base, &nvalid);
    const bool tree_tile = t >= np;

    // ---- two halves of 32 keys: S^T = K Q^T, online softmax, O^T += V^T P^T
    const bool need_mask = tree_tile || nvalid < kKeys;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      floatx16 sc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + kfrag0 + kb * (32 * kKRow + 4 * 64) + 32 * ks);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc, 0, 0, 0);
      }
      // mask (tree tiles and the ragged last prefix tile only) and row max.
      // Query rows past num_nodes need no masking: their scores never reach
      // a valid row and their outputs are written as zeros.
      float tmax = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * kb + 8 * gq + (v < 8 ? v : v + 8);
          const bool ok = kk < nvalid && (!tree_tile || ((mword >> kk) & 1ull) != 0);
          sc[v] = ok ? sc[v] : -INFINITY;
          tmax = fmaxf(tmax, sc[v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sc[v]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax * c_log2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      // P is carried as a pair of bf16 MFMA operands, P = hi + lo with
      // hi = bf16(p) and lo = bf16(p - hi): |p - hi - lo| <= 2^-18 p, so the
      // weights keep ~fp32 accuracy even when only a few keys contribute.
      float psum = 0.0f;
      bf16x8 pf[2], pl[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x2 hi2[4], lo2[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          floatx2 pr;
          pr[0] = __builtin_amdgcn_exp2f(fmaf(sc[8 * hf + 2 * e2], c_log2, -m_use));
          pr[1] = __builtin_amdgcn_exp2f(fmaf(sc[8 * hf + 2 * e2 + 1], c_log2, -m_use));
          psum += pr[0] + pr[1];
          hi2[e2] = __builtin_convertvector(pr, bf16x2);
          const uint32_t hb = __builtin_bit_cast(uint32_t, hi2[e2]);
          floatx2 rest = {pr[0] - __uint_as_float(hb << 16), pr[1] - __uint_as_float(hb & 0xFFFF0000u)};
          lo2[e2] = __builtin_convertvector(rest, bf16x2);
        }
        pf[hf] = bf16x8{hi2[0][0], hi2[0][1], hi2[1][0], hi2[1][1],
                        hi2[2][0], hi2[2][1], hi2[3][0], hi2[3][1]};
        pl[hf] = bf16x8{lo2[0][0], lo2[0][1], lo2[1][0], lo2[1][1],
                        lo2[2][0], lo2[2][1], lo2[3][0], lo2[3][1]};
      }
      l_run = l_run * alpha + psum;
      // the running max settles after a few tiles: rescale O only when it moved
      if (__ballot(m_new != m_run) != 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
      }
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int va = ((db & 1) ? (vfrag[2 * kb + hf] ^ 64) : vfrag[2 * kb + hf]) + db * 32 * kKeys * 2;
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vl + va);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[hf], acc_o[db], 0, 0, 0);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[hf], acc_o[db], 0, 0, 0);
        }
      }
    }
    if (has_next) write_tile(bf ^ 1);
    __syncthreads();
    bf ^= 1;
  }

  const float l_row = l_run + __shfl_xor(l_run, 32, 64);

  if (nsplit == 1) {
    if (row < R) {
      const float inv = (row_valid && l_row > 0.0f) ? 1.0f / l_row : 0.0f;
      uint16_t* o = O + (((size_t)b * T + node) * a.Hq + head) * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          floatx2 lo2 = {acc_o[db][4 * j] * inv, acc_o[db][4 * j + 1] * inv};
          floatx2 hi2 = {acc_o[db][4 * j + 2] * inv, acc_o[db][4 * j + 3] * inv};
          bf16x2 l2 = __builtin_convertvector(lo2, bf16x2);
          bf16x2 h2 = __builtin_convertvector(hi2, bf16x2);
          bf16x4 o4 = {l2[0], l2[1], h2[0], h2[1]};
          *reinterpret_cast<bf16x4*>(o + 32 * db + 8 * j + 4 * gq) = o4;
        }
      }
    }
    return;
  }

  // ---- split: write this split's partial (unnormalised O, m, l)
  const int Rpad = row_tiles * kTileRows;
  const size_t bh = (size_t)bhi;
  const size_t nbh = (size_t)a.batch * a.Hkv;
  {
    float* po = part_o + (((size_t)z * nbh + bh) * Rpad + row) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        floatx4 v4 = {acc_o[db][4 * j], acc_o[db][4 * j + 1], acc_o[db][4 * j + 2],
                      acc_o[db][4 * j + 3]};
        *reinterpret_cast<floatx4*>(po + 32 * db + 8 * j + 4 * gq) = v4;
      }
    if (gq == 0) {
      float* pm = part_ml + (((size_t)z * nbh + bh) * Rpad + row) * 2;
      pm[0] = m_run;
      pm[1] = l_row;
    }
  }
}

// Merge of the split partials: 32 query rows of one (request, kv-head) per
// workgroup. Per row, the split weights w_z = 2^(m_z - M) / sum_z 2^(m_z - M) l_z
// go to LDS; then each output chunk sums w_z O_z with several partial loads
// in flight per thread.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int nsplit, int row_tiles,
                                                      const float* part_o, const float* part_ml) {
  constexpr int kRows = 32;
  __shared__ float wts[kRows * 32];  // nsplit <= 32
  const int tid = threadIdx.x;
  const int b = blockIdx.y / a.Hkv, hk = blockIdx.y - (blockIdx.y / a.Hkv) * a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int T = a.T;
  const int R = T * g;
  const int nn = min(max(a.num_nodes[b], 0), T);
  const int nvalid_rows = nn * g;
  const int r0 = blockIdx.x * kRows;
  const int Rpad = row_tiles * kTileRows;
  const size_t bh = (size_t)b * a.Hkv + hk;
  const size_t nbh = (size_t)a.batch * a.Hkv;
  uint16_t* O = static_cast<uint16_t*>(a.out);
  // split maxima and sums of the 32 rows, all loads in flight at once
  __shared__ float sm[kRows * 32], sl[kRows * 32];
  const size_t zstride = nbh * Rpad * 2;
  for (int idx = tid; idx < kRows * nsplit; idx += 256) {
    const int rl = idx / nsplit, zz = idx - rl * nsplit;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + (bh * Rpad + r0 + rl) * 2 + zz * zstride);
    sm[idx] = ml.x;
    sl[idx] = ml.y;
  }
  __syncthreads();
  if (tid < kRows) {
    const int rr = r0 + tid;
    float M = -INFINITY;
    for (int zz = 0; zz < nsplit; ++zz) M = fmaxf(M, sm[tid * nsplit + zz]);
    float den = 0.f;
    for (int zz = 0; zz < nsplit; ++zz)
      den += (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[tid * nsplit + zz] - M) * sl[tid * nsplit + zz];
    const float inv = (den > 0.f && rr < nvalid_rows) ? 1.0f / den : 0.0f;
    for (int zz = 0; zz < nsplit; ++zz)
      wts[tid * nsplit + zz] = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[tid * nsplit + zz] - M) * inv;
  }
  __syncthreads();
  constexpr int kU = 8;
  for (int idx = tid; idx < kRows * (kD / 4); idx += 256) {
    const int rl = idx / (kD / 4), c4 = idx - rl * (kD / 4);
    const int rr = r0 + rl;
    if (rr >= R) continue;
    const int nd = rr / g, hd = hk * g + (rr - nd * g);
    const size_t pbase = (bh * Rpad + rr) * kD + 4 * c4;
    const size_t pstride = nbh * Rpad * kD;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z0 = 0; z0 < nsplit; z0 += kU) {
      float4 oz[kU];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int zz = min(z0 + j, nsplit - 1);
        oz[j] = *reinterpret_cast<const float4*>(part_o + pbase + zz * pstride);
      }
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const float wz = (z0 + j < nsplit) ? wts[rl * nsplit + z0 + j] : 0.f;
        acc.x += wz * oz[j].x;
        acc.y += wz * oz[j].y;
        acc.z += wz * oz[j].z;
        acc.w += wz * oz[j].w;
      }
    }
    floatx2 lo2 = {acc.x, acc.y}, hi2 = {acc.z, acc.w};
    bf16x2 l2 = __builtin_convertvector(lo2, bf16x2);
    bf16x2 h2 = __builtin_convertvector(hi2, bf16x2);
    bf16x4 o4 = {l2[0], l2[1], h2[0], h2[1]};
    *reinterpret_cast<bf16x4*>(O + (((size_t)b * T + nd) * a.Hq + hd) * kD + 4 * c4) = o4;
  }
}

// ------------------------------------------------------------------ fp32 path
template <typename IN_T>
__device__ __forceinline__ float load_f(const IN_T* p, size_t i) {
  if constexpr (sizeof(IN_T) == 2) return bf16_to_float(p[i]);
  else return p[i];
}

// One thread per query row (b, i, h); fp32 online softmax over the allowed keys.
template <typename IN_T, int D>
__global__ __launch_bounds__(128) void k_attn_simple(AttnArgs a) {
  const int64_t rid = (int64_t)blockIdx.x * 128 + threadIdx.x;
  const int64_t nrows = (int64_t)a.batch * a.T * a.Hq;
  if (rid >= nrows) return;
  const int h = (int)(rid % a.Hq);
  const int i = (int)((rid / a.Hq) % a.T);
  const int b = (int)(rid / ((int64_t)a.Hq * a.T));
  const IN_T* Q = static_cast<const IN_T*>(a.q);
  const IN_T* Kg = static_cast<const IN_T*>(a.k);
  const IN_T* Vg = static_cast<const IN_T*>(a.v);
  IN_T* O = static_cast<IN_T*>(a.out);
  const size_t obase = (((size_t)b * a.T + i) * a.Hq + h) * D;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  const int nn = min(max(a.num_nodes[b], 0), a.T);
  float l = 0.0f;
  if (i < nn) {
    float q[D];
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = load_f(Q, obase + d);
    const int g = a.Hq / a.Hkv, hk = h / g;
    const int P = max(a.prefix_lens[b], 0);
    const size_t kv0 = (size_t)a.kv_offsets[b];
    const int W = (a.T + 63) >> 6;
    const uint64_t* mrow = a.mask + ((size_t)b * a.T + i) * W;
    const float c = a.scale * kLog2e;
    float m = -INFINITY;
    for (int j = 0; j < P + nn; ++j) {
      if (j >= P) {
        const int t = j - P;
        if (((mrow[t >> 6] >> (t & 63)) & 1ull) == 0) continue;
      }
      if ((int64_t)(kv0 + j) >= a.total_rows) continue;
      const size_t kb = ((kv0 + j) * a.Hkv + hk) * D;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], load_f(Kg, kb + d), s);
      s *= c;
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, load_f(Vg, kb + d), acc[d] * alpha);
      m = mn;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float o = acc[d] * inv;
    if constexpr (sizeof(IN_T) == 2) {
      O[obase + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
    } else {
      O[obase + d] = o;
    }
  }
}

// Compute units of the current device (cached per device id).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    hipDeviceProp_t prop;
    cus[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                   ? prop.multiProcessorCount
                   : 256;
  }
  return cus[dev];
}

// Split of each row tile's key range across workgroups: pick the count that
// minimises a simple time model -- rounds of resident workgroups (two per
// CU) times the key tiles per workgroup, plus the partial-result traffic of
// the merge -- with at least 4 key tiles per split.
AttnSplit plan_split(int dtype, int batch, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  AttnSplit s{1, 0, 0, 0};
  if (dtype != 0 || D != kD) return s;
  const int g = Hq / Hkv;
  const int R = T * g;
  s.row_tiles = (R + kTileRows - 1) / kTileRows;
  const long blocks = (long)batch * Hkv * s.row_tiles;
  const int tiles = (max_prefix_len + kKeys - 1) / kKeys + (T + kKeys - 1) / kKeys;
  const long slots = 2L * device_cus();
  const double t_tile_us = 1.0, t_fixed_us = 3.0, hbm_bytes_per_us = 8.0e6;
  int best = 1;
  double best_t = 1e300;
  for (int ns = 1; ns <= 32; ++ns) {
    if (ns > 1 && tiles < 4 * ns) break;
    const long wgs = blocks * ns;
    const long rounds = (wgs + slots - 1) / slots;
    const int per = (tiles + ns - 1) / ns;
    double t = rounds * (per * t_tile_us + t_fixed_us);
    if (ns > 1) t += t_fixed_us + 2.0 * (double)wgs * kTileRows * kD * 4 / hbm_bytes_per_us;
    if (t < best_t * 0.97) {
      best_t = t;
      best = ns;
    }
  }
  s.nsplit = best;
  s.total = (int)(blocks * best);
  s.per_xcd = (s.total + kXcds - 1) / kXcds;
  return s;
}

template <typename IN_T>
hipError_t launch_simple(const AttnArgs& a, hipStream_t st) {
  const int64_t nrows = (int64_t)a.batch * a.T * a.Hq;
  dim3 grid((unsigned)((nrows + 127) / 128)), block(128);
  switch (a.D) {
    case 32: hipLaunchKernelGGL((k_attn_simple<IN_T, 32>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_attn_simple<IN_T, 64>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_attn_simple<IN_T, 128>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int dtype, int batch, int T, int Hq, int Hkv, int D,
                            int max_prefix_len) {
  const AttnSplit s = plan_split(dtype, batch, T, Hq, Hkv, D, max_prefix_len);
  if (s.nsplit <= 1) return 256;
  const size_t rows = (size_t)s.nsplit * batch * Hkv * s.row_tiles * kTileRows;
  return align_up(rows * kD * 4, 256) + align_up(rows * 2 * 4, 256);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  if (a.dtype == 1) return launch_simple<float>(a, st);
  if (a.D != kD) return launch_simple<uint16_t>(a, st);
  const AttnSplit s = plan_split(a.dtype, a.batch, a.T, a.Hq, a.Hkv, a.D, a.max_prefix_len);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (s.nsplit > 1) {
    const size_t rows = (size_t)s.nsplit * a.batch * a.Hkv * s.row_tiles * kTileRows;
    char* p = static_cast<char*>(ws);
    part_o = reinterpret_cast<float*>(p);
    p += align_up(rows * kD * 4, 256);
    part_ml = reinterpret_cast<float*>(p);
  }
  dim3 grid(s.per_xcd * kXcds), block(256);
  hipLaunchKernelGGL(k_attn_mfma, grid, block, 0, st, a, s, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.nsplit <= 1) return e;
  const int R = a.T * (a.Hq / a.Hkv);
  dim3 cgrid((R + 31) / 32, a.batch * a.Hkv);
  hipLaunchKernelGGL(k_attn_combine, cgrid, block, 0, st, a, s.nsplit, s.row_tiles,
                     (const float*)part_o, (const float*)part_ml);
  return hipGetLastError();
}

}  // namespace ddt
