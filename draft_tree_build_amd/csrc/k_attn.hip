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
// lists are split across workgroups and merged by the last split to arrive
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

// K tile: [64 keys][16 chunks of 8 dims]; chunk index XOR-swizzled by key so
// that the 8 lanes of a 128-bit LDS access hit distinct banks.
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
  int sw = (key & 3) | ((key >> 1) & 4);
  return key * (kD * 2) + ((chunk ^ sw) << 4);
}
// V^T tile: [128 dims][8 chunks of 8 keys]; chunk swizzled by dim.
__device__ __forceinline__ int v_lds_off(int dim, int chunk) {
  int sw = (dim ^ (dim >> 3)) & 7;
  return dim * (kKeys * 2) + ((chunk ^ sw) << 4);
}

struct AttnSplit {
  int nsplit;
  int row_tiles;
};

__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a, int nsplit, int row_tiles,
                                                      float* part_o, float* part_ml,
                                                      int32_t* counters) {
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[kKeys * kD * 2];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[kKeys * kD * 2];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int xt = blockIdx.x;
  const int b = blockIdx.y / a.Hkv, hk = blockIdx.y - (blockIdx.y / a.Hkv) * a.Hkv;
  const int z = blockIdx.z;
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
  auto tile_rows = [&](int t, int* base, int* nvalid) {
    if (t < np) {
      *base = t * kKeys;
      *nvalid = min(kKeys, P - t * kKeys);
    } else {
      const int tt = t - np;
      *base = P + tt * kKeys;
      *nvalid = min(kKeys, nn - tt * kKeys);
    }
  };
  auto load_tile = [&](int t) {
    int base, nvalid;
    tile_rows(t, &base, &nvalid);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + (j & 1) + 8 * (j >> 1);
      const int64_t kr = (int64_t)kv0 + base + key;
      const bool ok = key < nvalid && kr < a.total_rows;
      // out-of-range keys read row 0 (always valid) and are zeroed
      const size_t off = ((size_t)(ok ? kr : 0) * a.Hkv + hk) * kD + 8 * dc;
      const uint4 kx = *reinterpret_cast<const uint4*>(Kg + off);
      const uint4 vx = *reinterpret_cast<const uint4*>(Vg + off);
      sk[j] = ok ? kx : make_uint4(0, 0, 0, 0);
      sv[j] = ok ? vx : make_uint4(0, 0, 0, 0);
    }
  };

  // the key permutation of the S^T A operand: A row m -> key pi(m), chosen so
  // that lane group gq's score registers v = 0..7 hold keys 8 gq + v and
  // v = 8..15 hold keys 16 + 8 gq + (v - 8) of each 32-key block
  const int m_a = lane & 31;
  const int pi_m = 8 * ((m_a >> 2) & 1) + 16 * (m_a >> 4) + 4 * ((m_a >> 3) & 1) + (m_a & 3);

  for (int t = t_begin; t < t_end; ++t) {
    load_tile(t);
    __syncthreads();
    // K: 128-bit writes; V: transposed 32-bit writes of key pairs
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + (j & 1) + 8 * (j >> 1);
      *reinterpret_cast<uint4*>(k_lds + k_lds_off(key, dc)) = sk[j];
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
        *reinterpret_cast<uint32_t*>(v_lds + v_lds_off(dim, key >> 3) + (key & 7) * 2) = lo | hi;
      }
    }
    __syncthreads();

    int base, nvalid;
    tile_rows(t, &base, &nvalid);
    const bool tree_tile = t >= np;
    uint64_t mword = 0;
    if (tree_tile && row_valid) mword = a.mask[((size_t)b * T + node) * W + (t - np)];

    // ---- S^T = K Q^T for 2 blocks of 32 keys
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.0f;
      const int key = 32 * kb + pi_m;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(k_lds + k_lds_off(key, 2 * ks + gq));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---- mask, online softmax (log2 domain)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 32 * kb + 8 * gq + (v < 8 ? v : v + 8);
        const bool ok =
            row_valid && kk < nvalid && (!tree_tile || ((mword >> kk) & 1ull) != 0);
        const float x = ok ? s[kb][v] : -INFINITY;
        s[kb][v] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax * c_log2);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    // P is carried as a pair of bf16 MFMA operands, P = hi + lo with
    // hi = bf16(p) and lo = bf16(p - hi): |p - hi - lo| <= 2^-18 p, so the
    // weights keep ~fp32 accuracy even when only a few keys contribute.
    float psum = 0.0f;
    bf16x8 pf[2][2], pl[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x2 hi2[4], lo2[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          floatx2 pr;
          pr[0] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + 2 * e2], c_log2, -m_use));
          pr[1] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + 2 * e2 + 1], c_log2, -m_use));
          psum += pr[0] + pr[1];
          hi2[e2] = __builtin_convertvector(pr, bf16x2);
          const uint32_t hb = __builtin_bit_cast(uint32_t, hi2[e2]);
          floatx2 rest = {pr[0] - __uint_as_float(hb << 16), pr[1] - __uint_as_float(hb & 0xFFFF0000u)};
          lo2[e2] = __builtin_convertvector(rest, bf16x2);
        }
        pf[kb][hf] = bf16x8{hi2[0][0], hi2[0][1], hi2[1][0], hi2[1][1],
                            hi2[2][0], hi2[2][1], hi2[3][0], hi2[3][1]};
        pl[kb][hf] = bf16x8{lo2[0][0], lo2[0][1], lo2[1][0], lo2[1][1],
                            lo2[2][0], lo2[2][1], lo2[3][0], lo2[3][1]};
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = 32 * db + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(v_lds + v_lds_off(dim, 4 * kb + 2 * hf + gq));
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hf], acc_o[db], 0, 0, 0);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[kb][hf], acc_o[db], 0, 0, 0);
        }
      }
    }
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
  const size_t bh = (size_t)b * a.Hkv + hk;
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
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int ci = (int)(bh * row_tiles + xt);
    const int old = atomicAdd(&counters[ci], 1);
    s_last = (old == nsplit - 1) ? 1 : 0;
    if (s_last) counters[ci] = 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- last split: merge all splits of these 128 rows
  for (int idx = tid; idx < kTileRows * (kD / 4); idx += 256) {
    const int rl = idx / (kD / 4), c4 = idx - rl * (kD / 4);
    const int rr = tile_row0 + rl;
    if (rr >= R) continue;
    const int nd = rr / g, hd = hk * g + (rr - nd * g);
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rr < nvalid_rows) {
      float M = -INFINITY;
      for (int zz = 0; zz < nsplit; ++zz)
        M = fmaxf(M, part_ml[(((size_t)zz * nbh + bh) * Rpad + rr) * 2]);
      if (M != -INFINITY) {
        float den = 0.f;
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int zz = 0; zz < nsplit; ++zz) {
          const size_t pr = ((size_t)zz * nbh + bh) * Rpad + rr;
          const float mz = part_ml[pr * 2];
          const float wz = __builtin_amdgcn_exp2f(mz - M);  // 0 for an empty split
          den += wz * part_ml[pr * 2 + 1];
          const float4 oz = *reinterpret_cast<const float4*>(part_o + pr * kD + 4 * c4);
          num.x += wz * oz.x;
          num.y += wz * oz.y;
          num.z += wz * oz.z;
          num.w += wz * oz.w;
        }
        const float inv = den > 0.f ? 1.0f / den : 0.0f;
        res = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
      }
    }
    floatx2 lo2 = {res.x, res.y}, hi2 = {res.z, res.w};
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

AttnSplit plan_split(int dtype, int batch, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  AttnSplit s{1, 0};
  if (dtype != 0 || D != kD) return s;
  const int g = Hq / Hkv;
  const int R = T * g;
  s.row_tiles = (R + kTileRows - 1) / kTileRows;
  const long blocks = (long)batch * Hkv * s.row_tiles;
  const int tiles = (max_prefix_len + kKeys - 1) / kKeys + (T + kKeys - 1) / kKeys;
  const long target = 512;
  int ns = (int)((target + blocks - 1) / blocks);
  ns = std::min(ns, std::max(1, tiles / 4));
  ns = std::max(1, std::min(ns, 32));
  s.nsplit = ns;
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
  return align_up(rows * kD * 4, 256) + align_up(rows * 2 * 4, 256) +
         align_up((size_t)batch * Hkv * s.row_tiles * 4, 256);
}

hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  if (a.dtype == 1) return launch_simple<float>(a, st);
  if (a.D != kD) return launch_simple<uint16_t>(a, st);
  const AttnSplit s = plan_split(a.dtype, a.batch, a.T, a.Hq, a.Hkv, a.D, a.max_prefix_len);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int32_t* counters = nullptr;
  if (s.nsplit > 1) {
    const size_t rows = (size_t)s.nsplit * a.batch * a.Hkv * s.row_tiles * kTileRows;
    char* p = static_cast<char*>(ws);
    part_o = reinterpret_cast<float*>(p);
    p += align_up(rows * kD * 4, 256);
    part_ml = reinterpret_cast<float*>(p);
    p += align_up(rows * 2 * 4, 256);
    counters = reinterpret_cast<int32_t*>(p);
  }
  dim3 grid(s.row_tiles, a.batch * a.Hkv, s.nsplit), block(256);
  hipLaunchKernelGGL(k_attn_mfma, grid, block, 0, st, a, s.nsplit, s.row_tiles, part_o, part_ml,
                     counters);
  return hipGetLastError();
}

}  // namespace ddt
