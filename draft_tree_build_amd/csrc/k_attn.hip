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
// of 64 rows go from HBM straight into LDS by DMA (global_load_lds, no
// registers), row-major with an XOR swizzle of the 16-byte chunks. Per wave
// and tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16
// (lane = query row), online softmax in fp32 (exp2 domain) against a
// running reference that moves only when the weights would leave the fp16
// range, O^T += V^T P^T on v_mfma_f32_32x32x16_f16 with P as fp16 (2^-11
// relative per weight, against 2^-8 for bf16 weights). V enters as fp16 in
// fragment order -- each MFMA operand fragment one 16-byte load per lane:
// every wave converts the V rows it staged once, taking them out transposed
// through ds_read_b64_tr_b16 and writing them back in that order, or, when
// many row tiles read every V tile, a pass of its own (k_v_f16) writes the
// request's V tiles so once before the main kernel, which then copies each
// tile as one block. A row tile of
// at most 32 rows has two waves take its keys by 32-key halves. The key tile
// list is prefix tiles then tree tiles (mask applied); long lists are split
// across workgroups and merged by a second kernel (log-sum-exp weights).
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

// K and V tiles: 64 rows of 256 bytes (128 dims) at row * 256; the 16-byte
// chunk c of row r sits at physical chunk c ^ sw(r), sw(r) = the low four
// row bits with their two pairs swapped. Measured on gfx950 (LDS bank
// conflict counter), this keeps both the K fragment reads (16 keys, one
// chunk each) and the V transpose reads (4 consecutive keys, 2 chunks each)
// free of bank conflicts. A V tile is then rewritten in fragment order
// (v_tile_to_frag).
constexpr int kTileBytes = kKeys * kD * 2;  // 16 KB
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * 256 + ((chunk ^ swz(row)) << 4); }

// V fragments, the A operand of O^T += V^T P^T on v_mfma_f32_32x32x16_f16:
// for dims 32 db .. + 31 and keys 16 s .. + 15 of a tile, lane l holds
// dim 32 db + l % 32 and keys 16 s + 8 (l / 32) + 0..7. From a row-major
// tile they come out transposed through two ds_read_b64_tr_b16 (4 keys
// each): 16-lane group G holds dims 32 db + 16 (G % 2) + 0..15 and keys
// 16 s + 8 (G / 2) + 0..7; read rd covers keys + 4 rd .. + 3, lane i of the
// group pointing at key + i / 4, dims + 4 (i % 4) .. + 3. v_tr_off is that
// pointer's byte offset for keys 16 s = 0; key step s adds s * 16 rows.
__device__ __forceinline__ int v_tr_off(int lane, int db, int rd) {
  const int G = lane >> 4, ti = lane & 15;
  const int row = 8 * (G >> 1) + 4 * rd + (ti >> 2);
  const int dim = 32 * db + 16 * (G & 1) + 4 * (ti & 3);
  return tile_off(row, dim >> 3) + ((dim & 7) << 1);
}
__device__ __forceinline__ halfx8 v_frag_tr(const unsigned char* p0, const unsigned char* p1) {
  const v4s v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p0);
  const v4s v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p1);
  return __builtin_bit_cast(halfx8, (short8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
}

// bf16 -> fp16 for key step s = w of a V tile -- the 16 rows that wave w
// staged, bytes 4096 w .. 4096 w + 4095, row-major -- rewritten in place in
// fragment order: the fragment of dims 32 db .. + 31 at (4 w + db) * 1024,
// lane l's 16 bytes at 16 l (the layout k_v_f16 writes). The conversion is
// exact for |v| in [2^-14, 65504]; smaller values round to fp16 subnormals
// (absolute error <= 2^-25). Called after the wave's own DMA has landed and
// before the barrier that publishes the tile. vtr[db][rd] = v_tr_off(lane,
// db, rd).
__device__ __forceinline__ void v_tile_to_frag(unsigned char* vbuf, int w, int lane, const int (&vtr)[4][2]) {
  const unsigned char* rows = vbuf + w * 16 * 256;
  halfx8 f[4];  // bf16 bit patterns
#pragma unroll
  for (int db = 0; db < 4; ++db) f[db] = v_frag_tr(rows + vtr[db][0], rows + vtr[db][1]);
  // every read of the wave before any write: the writes cover rows that
  // other lanes read
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const uint4 u = __builtin_bit_cast(uint4, f[db]);
    const uint32_t in[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx2 x = {__uint_as_float(in[q] << 16), __uint_as_float(in[q] & 0xFFFF0000u)};
      o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, halfx2));
    }
    *reinterpret_cast<uint4*>(vbuf + (4 * w + db) * 1024 + 16 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Request b's key rows kv0 .. kv0 + P + T must lie inside the caches; the
// offsets and lengths may come from earlier kernels, so this is checked here.
__device__ __forceinline__ bool kv_in_range(int64_t kv0, int P, int T, int64_t total_rows) {
  return kv0 >= 0 && P >= 0 && kv0 <= total_rows - (int64_t)P - T;
}

__device__ __forceinline__ void set_status(int32_t* status, int b, int bits) {
  if (status) atomicOr(status + b, bits);
}

constexpr int kStatusNonfinite = 4;  // DDTREE_STATUS_OUT_NONFINITE
constexpr int kStatusBadKv = 8;      // DDTREE_STATUS_BAD_KV

struct AttnSplit {
  int nsplit;
  int row_tiles;
  int chunk;        // splits per unit
  int unit_chunks;  // units per (request, kv-head): ceil(nsplit / chunk)
  int units;        // batch * Hkv * unit_chunks
  int per_xcd;      // workgroups per XCD: ceil(units / 8) * chunk * row_tiles
  int preconv;      // V converted to fp16 once per request before the main kernel
};

// V is converted to fp16 by a separate pass (k_v_f16) when this many row
// tiles or more read every K/V tile: each of them would otherwise convert
// its V tiles again (measured: the in-kernel conversion costs 8.6% of the
// verify at 33 row tiles; the pass moves the request's V bytes twice).
constexpr int kPreconvMinRowTiles = 16;
constexpr size_t kPreconvMaxBytes = (size_t)4 << 30;

// Key tiles of one (request, kv-head) in the fp16 V copy: the prefix tiles
// of the longest prefix, then the tree tiles.
__host__ __device__ inline int vh_tiles(int T, int max_prefix_len) {
  return (int)(((long long)max_prefix_len + kKeys - 1) / kKeys + ((long long)T + kKeys - 1) / kKeys);
}

// fp16 copy of the V tiles the verify reads, with the same rounding as
// v_tile_to_frag, laid out in fragment order: key tile t of (request b,
// kv-head h) is 16 KB at vh + ((b * Hkv + h) * vh_tiles + t) * 16384 bytes
// -- t numbers the tiles as the main kernel does (prefix tiles, then tree
// tiles from key P_b on) -- and holds the 16 V fragments of the tile, key
// step s = 0..3 and dim block db = 0..3 at (4 s + db) * 1024, lane l's 16
// bytes at 16 l. The main kernel thus stages a tile with one contiguous
// copy and reads each fragment with one ds_read_b128 free of bank
// conflicts. Keys a tile does not hold (past the prefix, past num_nodes)
// are zeros. Requests outside the caches or with P_b > max_prefix_len are
// skipped (the main kernel converts those itself). One workgroup per tile;
// grid: x = tile, y = kv-head, z = request.
__global__ __launch_bounds__(256) void k_v_f16(AttnArgs a, uint16_t* vh) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kTileBytes];
  const int t = (int)blockIdx.x, hk = (int)blockIdx.y, b = (int)blockIdx.z;
  const int64_t kv0 = a.kv_offsets[b];
  const int P = a.prefix_lens[b];
  const int T = a.T;
  if (!kv_in_range(kv0, P, T, a.total_rows) || P > a.max_prefix_len) return;
  const int np = (P + kKeys - 1) / kKeys;
  if (t >= np + (T + kKeys - 1) / kKeys) return;
  int base, nvalid;
  if (t < np) {
    base = t * kKeys;
    nvalid = min(kKeys, P - base);
  } else {
    const int tt = t - np;
    base = P + tt * kKeys;
    nvalid = min(kKeys, min(max(a.num_nodes[b], 0), T) - tt * kKeys);
  }
  // rows base .. base + nvalid - 1 lie inside the request's P_b + T rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned char* src = reinterpret_cast<const unsigned char*>(a.v) +
                             ((size_t)(kv0 + base) * a.Hkv + hk) * (kD * 2);
  const size_t row_bytes = (size_t)a.Hkv * kD * 2;
  // row-major, swizzled, converted: wave w takes rows 16 w .. 16 w + 15
  uint4 u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * (4 * w + j) + (lane >> 4);
    const int c = (lane & 15) ^ swz(r);
    u[j] = r < nvalid ? *reinterpret_cast<const uint4*>(src + r * row_bytes + c * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t in[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx2 f = {__uint_as_float(in[q] << 16), __uint_as_float(in[q] & 0xFFFF0000u)};
      o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, halfx2));
    }
    *reinterpret_cast<uint4*>(lds + (4 * w + j) * 1024 + 16 * lane) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
  // wave w writes the fragments of key step s = w
  unsigned char* dst = reinterpret_cast<unsigned char*>(vh) +
                       (((size_t)b * a.Hkv + hk) * vh_tiles(T, a.max_prefix_len) + t) * kTileBytes;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const unsigned char* p = lds + w * 16 * 256;
    const halfx8 f = v_frag_tr(p + v_tr_off(lane, db, 0), p + v_tr_off(lane, db, 1));
    *reinterpret_cast<halfx8*>(dst + (4 * w + db) * 1024 + 16 * lane) = f;
  }
}

constexpr int kXcds = 8;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// One workgroup = 128 query rows of one (request, kv-head) over one range of
// key tiles. Grid: 1-D, XCD-aware -- consecutive workgroup ids go to
// different XCDs, so XCD x runs workgroups x, x + 8, ... Units of work --
// one (request, kv-head) with a run of `chunk` consecutive splits, all their
// row tiles -- are dealt to the XCDs in turn, unit u to XCD u % 8: the row
// tiles of a split share its K/V tiles in one L2, the splits of a unit share
// its Q rows, and every request is spread over the XCDs, which keeps them
// evenly loaded when prefix lengths differ. Splits are cut into several
// units only when there are fewer (request, kv-head) pairs than XCDs. Key
// tiles are double-buffered in LDS: tile t+1 is copied into the other buffer
// while tile t is computed.
__global__ __launch_bounds__(256, 2) void k_attn_mfma(AttnArgs a, AttnSplit pl, float* part_o,
                                                      float* part_ml, const uint16_t* vh) {
  // two buffers of K and V tiles; 64 KB
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds1[kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nsplit = pl.nsplit, row_tiles = pl.row_tiles;
  const int xj = (int)(blockIdx.x / kXcds);  // this workgroup's place on its XCD
  const int per_unit = pl.chunk * row_tiles;
  const int u = (xj / per_unit) * kXcds + (int)(blockIdx.x % kXcds);  // unit
  const int in_unit = xj % per_unit;
  const int z = (u % pl.unit_chunks) * pl.chunk + in_unit / row_tiles;
  if (u >= pl.units || z >= nsplit) return;
  const int xt = in_unit % row_tiles;
  const int bhi = u / pl.unit_chunks;
  const int hk = bhi % a.Hkv;
  // Requests are taken longest prefix first (ties: lower index first), so
  // that on every XCD the longest workgroups start first and the short ones
  // fill the tail. Every workgroup ranks the prefix lengths the same way:
  // lane i holds request i's length and counts the requests ahead of it.
  int b = bhi / a.Hkv;
  if (a.batch > 1 && a.batch <= 64) {
    const int pl_i = lane < a.batch ? max(a.prefix_lens[lane], 0) : -1;
    int ahead = 0;
    for (int j = 0; j < a.batch; ++j) {
      const int pl_j = __builtin_amdgcn_readlane(pl_i, j);
      ahead += (pl_j > pl_i || (pl_j == pl_i && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < a.batch && ahead == b);
    b = __ffsll((unsigned long long)hit) - 1;
  }
  const int g = a.Hq / a.Hkv;
  const int T = a.T;
  const int R = T * g;
  const int64_t kv0s = a.kv_offsets[b];
  const int P = a.prefix_lens[b];
  const bool kv_ok = kv_in_range(kv0s, P, T, a.total_rows);
  // a request outside the caches reads no key: all its rows are padding
  const int nn = kv_ok ? min(max(a.num_nodes[b], 0), T) : 0;
  const int nvalid_rows = nn * g;
  const int tile_row0 = xt * kTileRows;
  if (!kv_ok && z == 0 && xt == 0 && tid == 0) set_status(a.status, b, kStatusBadKv);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v);
  uint16_t* O = static_cast<uint16_t*>(a.out);

  // A last row tile of at most 32 rows -- the last node's g heads when
  // T = N + 1 -- would leave three waves on padding rows. There waves 0 and
  // 1 take the same 32 rows, each one 32-key half of every key tile, and
  // merge their partial results at the end; waves 2 and 3 only stage tiles.
  const bool halves = R - tile_row0 <= kRowsPerWave;

  // rows of this lane: query row n = lane % 32 of wave w
  const int gq = lane >> 5;           // lane group (0/1)
  const int n = lane & 31;
  const int row = tile_row0 + (halves ? 0 : w * kRowsPerWave) + n;
  const int node = row / g;
  const int head = hk * g + (row - node * g);
  const bool row_valid = row < nvalid_rows;

  if (tile_row0 >= nvalid_rows) {
    // padding rows only: split 0 writes the zeros
    if (z == 0 && row < R && (!halves || w == 0)) {
      uint16_t* o = O + (((size_t)b * T + node) * a.Hq + head) * kD;
      for (int c = gq; c < kD / 8; c += 2) reinterpret_cast<uint4*>(o)[c] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  // ---- key tiles of this row tile: prefix tiles then tree tiles
  const int np = (P + kKeys - 1) / kKeys;
  const int last_row = min(tile_row0 + kTileRows, nvalid_rows) - 1;
  const int max_node = last_row / g;  // ancestors have smaller indices
  const int nt = (max_node + 1 + kKeys - 1) / kKeys;
  const int ntiles = np + nt;
  const int per = (ntiles + nsplit - 1) / nsplit;
  const int t_begin = min(z * per, ntiles), t_end = min(t_begin + per, ntiles);
  const size_t kv0 = (size_t)kv0s;
  // V tiles come converted to fp16, in fragment order, from k_v_f16 when it
  // ran for this request. The rest of the kernel is compiled once for each
  // case, so that neither carries a branch on it inside the tile loop
  // (measured: such branches cost 6-10% of the verify, since they cut the
  // schedule of LDS reads, exponentials and MFMAs into pieces).
  auto rest = [&](auto pre_tag) __attribute__((always_inline)) {
    constexpr bool pre = decltype(pre_tag)::value;
    const unsigned char* vh_bh =
        pre ? reinterpret_cast<const unsigned char*>(vh) +
                  ((size_t)b * a.Hkv + hk) * vh_tiles(T, a.max_prefix_len) * kTileBytes
            : nullptr;
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
    // padding rows (no keys, zero Q) take a finite reference from the start
    float m_run = row_valid ? -INFINITY : 0.0f, l_run = 0.0f;

    // ---- staging by DMA: wave w moves rows 16 w .. 16 w + 15 of K and V, four
    // 1 KB blocks each; lane i of a block writes LDS bytes 16 i of it, so it
    // fetches row 4 blk + i / 16, logical chunk (i % 16) ^ sw(row).
    const uint32_t row_bytes = (uint32_t)a.Hkv * kD * 2;
    uint32_t dma_off[4];   // byte offset from the tile's first K/V row
    int dma_row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * w + j;
      const int r = 4 * blk + (lane >> 4);
      const int c = (lane & 15) ^ swz(r);
      dma_row[j] = r;
      dma_off[j] = (uint32_t)r * row_bytes + (uint32_t)hk * (kD * 2) + (uint32_t)c * 16;
    }
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
    auto dma_tile = [&](int t, unsigned char* kbuf, unsigned char* vbuf) __attribute__((always_inline)) {
      int base, nvalid;
      tile_rows(t, &base, &nvalid);
      // every key row of the request is inside the caches (kv_in_range) and a
      // tile holds at least one valid key
      const size_t tb = (kv0 + (size_t)base) * row_bytes;
      const unsigned char* kt = reinterpret_cast<const unsigned char*>(Kg) + tb;
      const unsigned char* vt = reinterpret_cast<const unsigned char*>(Vg) + tb;
      // the fp16 copy's tile is one contiguous 16 KB block, copied as it is
      const unsigned char* vp = pre ? vh_bh + (size_t)t * kTileBytes + (4 * w) * 1024 + 16 * lane : nullptr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows past the tile's nvalid keys re-read the tile's first row: their
        // scores are masked (allow covers keys < nvalid only), so they only
        // ever meet zero weights
        const uint32_t off = dma_row[j] < nvalid ? dma_off[j] : dma_off[j] - (uint32_t)dma_row[j] * row_bytes;
        unsigned char* kd = kbuf + (4 * w + j) * 1024;
        unsigned char* vd = vbuf + (4 * w + j) * 1024;
        __builtin_amdgcn_global_load_lds(kt + off, (__attribute__((address_space(3))) void*)kd, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(pre ? vp + j * 1024 : vt + off,
                                         (__attribute__((address_space(3))) void*)vd, 16, 0, 0);
      }
    };

    // ---- fragment addresses (bytes within a tile)
    // K (A operand of S^T): lane row m -> key pi(m), chosen so that lane group
    // gq's score registers v = 0..7 hold keys 8 gq + v and v = 8..15 hold keys
    // 16 + 8 gq + (v - 8) of each 32-key half; dims 16 ks + 8 gq + 0..7.
    const int m_a = lane & 31;
    const int pi_m = 8 * ((m_a >> 2) & 1) + 16 * (m_a >> 4) + 4 * ((m_a >> 3) & 1) + (m_a & 3);
    int kfrag[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kfrag[ks] = tile_off(pi_m, 2 * ks + gq);
    // V fragments from a row-major tile (key step 0; see v_tr_off), for the
    // in-kernel conversion
    int vfrag[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) vfrag[db][rd] = v_tr_off(lane, db, rd);

    // mask word of this lane's query row for tree tile t (prefetched with the tile)
    const uint64_t* mrow = a.mask + ((size_t)b * T + node) * W;
    auto load_mword = [&](int t) __attribute__((always_inline)) -> uint64_t {
      return (t >= np && row_valid) ? mrow[t - np] : 0ull;
    };
    // V fragments (A operand of O^T += V^T P^T) of 32-key half kb of the tile
    // in vl, which is in fragment order: key steps s = 2 kb + hf, one
    // 16-byte read each
    auto read_v = [&](const unsigned char* vl, int kb, halfx8 (&vf)[4][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          vf[db][hf] = *reinterpret_cast<const halfx8*>(vl + (4 * (2 * kb + hf) + db) * 1024 + 16 * lane);
    };
    // Scores of 32-key half kb masked to the allowed keys (tree tiles and the
    // ragged last prefix tile). Query rows past num_nodes need no masking:
    // their scores never reach a valid row and their outputs are written as
    // zeros.
    auto apply_mask = [&](floatx16& s, uint64_t allow, int kb) __attribute__((always_inline)) {
      // register v holds key 32 kb + 8 gq + v (v < 8) or + 8 more (v >= 8)
      const uint32_t sh = 32 * kb + 8 * gq;
      const uint32_t bits = (uint32_t)((allow >> sh) & 0xFFull) | ((uint32_t)((allow >> (sh + 16)) & 0xFFull) << 8);
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = ((bits >> v) & 1u) ? s[v] : -INFINITY;
    };
    // Weights p = 2^(s c - m_run) of one half against the row's reference
    // m_run, taken without a maximum. The reference is an exact running
    // maximum of the row's scores, re-taken only where it has to move: on a
    // half tile whose weights sum to more than 2^15 (or to no finite value),
    // and while a row has met no key (m_run = -inf). Weights then stay below
    // 2^15, inside fp16; O and l share the reference, so O / l is unchanged.
    // The row sum l adds the fp16 weights that enter the P.V product
    // (v_dot2_f32_f16 with fp32 accumulation).
    auto probs = [&](const floatx16& s, halfx8 (&pf)[2]) __attribute__((always_inline)) -> float {
      const float neg_m = (m_run == -INFINITY) ? 0.0f : -m_run;
      float ps = 0.0f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        halfx2 h2[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          floatx2 pr;
          pr[0] = __builtin_amdgcn_exp2f(fmaf(s[8 * hf + 2 * e2], c_log2, neg_m));
          pr[1] = __builtin_amdgcn_exp2f(fmaf(s[8 * hf + 2 * e2 + 1], c_log2, neg_m));
          h2[e2] = __builtin_convertvector(pr, halfx2);
          ps = __builtin_amdgcn_fdot2(h2[e2], halfx2{(_Float16)1.0f, (_Float16)1.0f}, ps, false);
        }
        pf[hf] = halfx8{h2[0][0], h2[0][1], h2[1][0], h2[1][1], h2[2][0], h2[2][1], h2[3][0], h2[3][1]};
      }
      return ps;
    };
    // the rare path: the half tile's exact maximum becomes the reference
    // where it is larger, O and l are rescaled, the weights recomputed
    auto settle = [&](const floatx16& s, halfx8 (&pf)[2], float& ps) __attribute__((always_inline)) {
      if (__ballot(m_run == -INFINITY || !(ps <= 32768.0f)) == 0ull) return;
      float hmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) hmax = fmaxf(hmax, s[v]);
      hmax = fmaxf(hmax, __shfl_xor(hmax, 32, 64));
      const float m_new = fmaxf(m_run, hmax * c_log2);
      const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      ps = probs(s, pf);
    };
    auto pv = [&](const halfx8 (&vfr)[4][2], const halfx8 (&pf)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfr[db][hf], pf[hf], acc_o[db], 0, 0, 0);
    };
    // allowed keys of this lane's query row in tile t: in range and (tree
    // tiles) ancestors
    auto tile_allow = [&](int t, uint64_t mword, bool* need_mask) __attribute__((always_inline)) -> uint64_t {
      int base, nvalid;
      tile_rows(t, &base, &nvalid);
      const bool tree_tile = t >= np;
      *need_mask = tree_tile || nvalid < kKeys;
      uint64_t allow = nvalid >= kKeys ? ~0ull : ((1ull << nvalid) - 1ull);
      if (tree_tile) allow &= mword;
      return allow;
    };

    // One key tile from LDS (kl, vl: the tile's K and V buffers; nk, nv: the
    // other buffers, where the next tile's DMA goes when has_next). Both
    // 32-key halves of S^T are computed first (two independent MFMA chains);
    // the weights of each half are then taken against the row's running
    // reference, and the exponentials of the second half run on the VALU
    // while the first half's O^T += V^T P^T products occupy the matrix core.
    uint64_t mword_next = 0;
    auto tile_body = [&](int t, uint64_t mword, const unsigned char* kl, const unsigned char* vl,
                         unsigned char* nk, unsigned char* nv, bool has_next)
        __attribute__((always_inline)) {
      bool need_mask;
      const uint64_t allow = tile_allow(t, mword, &need_mask);

      // ---- S^T = K Q^T for keys 0..31 (sc[0]) and 32..63 (sc[1])
      floatx16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[kb][v] = 0.0f;
      // K fragments read two steps ahead of their MFMAs (four in flight)
      bf16x8 kf[8][2];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kf[ks][kb] = *reinterpret_cast<const bf16x8*>(kl + kfrag[ks] + kb * 32 * 256);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][kb], qf[ks], sc[kb], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // the next tile's DMA is issued while the score MFMAs run
      if (has_next) {
        dma_tile(t + 1, nk, nv);
        mword_next = load_mword(t + 1);
      }
      // V fragments of the first half, read while the scores are computed
      halfx8 vf[4][2];
      read_v(vl, 0, vf);
      if (need_mask) {
        apply_mask(sc[0], allow, 0);
        apply_mask(sc[1], allow, 1);
      }
      halfx8 pf0[2];
      float ps0 = probs(sc[0], pf0);
      settle(sc[0], pf0, ps0);
      pv(vf, pf0);
      l_run += ps0;
      halfx8 vf1[4][2];
      read_v(vl, 1, vf1);
      halfx8 pf1[2];
      float ps1 = probs(sc[1], pf1);
      settle(sc[1], pf1, ps1);
      pv(vf1, pf1);
      l_run += ps1;
    };
    // The same tile when waves 0 and 1 share 32 rows (halves): wave w takes
    // the keys of half w; waves 2 and 3 only stage their part of the next tile.
    auto half_body = [&](int t, uint64_t mword, const unsigned char* kl, const unsigned char* vl,
                         unsigned char* nk, unsigned char* nv, bool has_next)
        __attribute__((always_inline)) {
      if (w >= 2) {
        if (has_next) dma_tile(t + 1, nk, nv);
        return;
      }
      bool need_mask;
      const uint64_t allow = tile_allow(t, mword, &need_mask);
      floatx16 s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.0f;
      bf16x8 kf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kl + kfrag[ks] + w * 32 * 256);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
      if (has_next) {
        dma_tile(t + 1, nk, nv);
        mword_next = load_mword(t + 1);
      }
      halfx8 vf[4][2];
      read_v(vl, w, vf);
      if (need_mask) apply_mask(s, allow, w);
      halfx8 pf[2];
      float ps = probs(s, pf);
      settle(s, pf, ps);
      pv(vf, pf);
      l_run += ps;
    };

    // Tiles alternate between two LDS buffers (static, so that the compiler
    // sees the DMA into one buffer and the reads of the other as disjoint):
    // while tile t is computed from one buffer, tile t+1 lands in the other.
    auto run_tiles = [&](auto&& body) __attribute__((always_inline)) {
      if (t_begin < t_end) {
        dma_tile(t_begin, k_lds0, v_lds0);
        mword_next = load_mword(t_begin);
      }
      __builtin_amdgcn_s_waitcnt(0);
      if (t_begin < t_end && !pre) v_tile_to_frag(v_lds0, w, lane, vfrag);
      __syncthreads();
      for (int t = t_begin; t < t_end; t += 2) {
        {
          const uint64_t mword = mword_next;
          body(t, mword, k_lds0, v_lds0, k_lds1, v_lds1, t + 1 < t_end);
          __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA of tile t+1 has landed
          if (t + 1 < t_end && !pre) v_tile_to_frag(v_lds1, w, lane, vfrag);
          __syncthreads();
        }
        if (t + 1 < t_end) {
          const uint64_t mword = mword_next;
          body(t + 1, mword, k_lds1, v_lds1, k_lds0, v_lds0, t + 2 < t_end);
          __builtin_amdgcn_s_waitcnt(0);
          if (t + 2 < t_end && !pre) v_tile_to_frag(v_lds0, w, lane, vfrag);
          __syncthreads();
        }
      }
    };
    if (!halves) {
      run_tiles(tile_body);
    } else {
      run_tiles(half_body);
      // wave 1 hands its (m, l, O) to wave 0 through the idle K buffer; each
      // lane's rows are the same in both waves, so the merge is per lane:
      // M = max(m0, m1), O = O0 2^(m0 - M) + O1 2^(m1 - M), l likewise
      float* xo = reinterpret_cast<float*>(k_lds0);  // 64 values per lane: 16 KB
      float* xm = reinterpret_cast<float*>(v_lds0);
      if (w == 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) xo[(db * 16 + v) * 64 + lane] = acc_o[db][v];
        xm[lane] = m_run;
        xm[64 + lane] = l_run;
      }
      __syncthreads();
      if (w != 0) return;
      const float m1 = xm[lane], l1 = xm[64 + lane];
      const float mm = fmaxf(m_run, m1);
      const float a0 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mm);
      const float a1 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] = acc_o[db][v] * a0 + xo[(db * 16 + v) * 64 + lane] * a1;
      l_run = l_run * a0 + l1 * a1;
      m_run = mm;
    }

    const float l_row = l_run + __shfl_xor(l_run, 32, 64);

    if (nsplit == 1) {
      bool bad = false;
      if (row < R) {
        const float inv = (row_valid && l_row > 0.0f) ? 1.0f / l_row : 0.0f;
        uint16_t* o = O + (((size_t)b * T + node) * a.Hq + head) * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            floatx2 lo2 = {acc_o[db][4 * j] * inv, acc_o[db][4 * j + 1] * inv};
            floatx2 hi2 = {acc_o[db][4 * j + 2] * inv, acc_o[db][4 * j + 3] * inv};
            bad |= !__builtin_isfinite(lo2[0]) | !__builtin_isfinite(lo2[1]) |
                   !__builtin_isfinite(hi2[0]) | !__builtin_isfinite(hi2[1]);
            bf16x2 l2 = __builtin_convertvector(lo2, bf16x2);
            bf16x2 h2 = __builtin_convertvector(hi2, bf16x2);
            bf16x4 o4 = {l2[0], l2[1], h2[0], h2[1]};
            *reinterpret_cast<bf16x4*>(o + 32 * db + 8 * j + 4 * gq) = o4;
          }
        }
      }
      // a non-finite output (an infinite fp16 V value, or a non-finite input)
      // is reported once per wave
      if (__ballot(bad) != 0ull && lane == 0) set_status(a.status, b, kStatusNonfinite);
      return;
    }

    // ---- split: write this split's partial (unnormalised O, m, l), streamed
    // past the L2 (nontemporal): read once by the merge kernel, they would
    // otherwise wait dirty in L2 for the end-of-kernel write-back (measured:
    // 16.5 -> 14.9 us at a 2048-key prefix, merge 4.0 -> 4.3 us)
    const int Rpad = row_tiles * kTileRows;
    const size_t bh = (size_t)b * a.Hkv + hk;  // the merge reads (request, kv-head)
    const size_t nbh = (size_t)a.batch * a.Hkv;
    if (row_valid) {  // rows past num_nodes are zeroed by the merge, which never reads them
      float* po = part_o + (((size_t)z * nbh + bh) * Rpad + row) * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          floatx4 v4 = {acc_o[db][4 * j], acc_o[db][4 * j + 1], acc_o[db][4 * j + 2],
                        acc_o[db][4 * j + 3]};
          __builtin_nontemporal_store(v4, reinterpret_cast<floatx4*>(po + 32 * db + 8 * j + 4 * gq));
        }
      if (gq == 0) {
        float* pm = part_ml + (((size_t)z * nbh + bh) * Rpad + row) * 2;
        __builtin_nontemporal_store(m_run, pm);
        __builtin_nontemporal_store(l_row, pm + 1);
      }
    }
  };
  if (vh != nullptr && P <= a.max_prefix_len)
    rest(BoolTag<true>{});
  else
    rest(BoolTag<false>{});
}

// Merge of the split partials: 8 query rows of one (request, kv-head) per
// workgroup, one 16-byte output chunk per thread. Per row, the split weights
// are w_z = 2^(m_z - M) / sum_z 2^(m_z - M) l_z (M = max_z m_z); each thread
// requests its row's (m_z, l_z) and its chunk of every O_z together (eight
// splits per round trip), computes the weights itself and sums w_z O_z.
// Rows past num_nodes have no partials: they are written as zeros.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int nsplit, int row_tiles,
                                                      const float* part_o, const float* part_ml) {
  constexpr int kRows = 8;
  constexpr int kU = 8;  // splits per round trip
  const int tid = threadIdx.x;
  const int rl = tid >> 5, c4 = tid & 31;
  const int b = blockIdx.y / a.Hkv, hk = blockIdx.y - (blockIdx.y / a.Hkv) * a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int T = a.T;
  const int R = T * g;
  const int rr = blockIdx.x * kRows + rl;
  if (rr >= R) return;
  const bool kv_ok = kv_in_range(a.kv_offsets[b], a.prefix_lens[b], T, a.total_rows);
  const int nn = kv_ok ? min(max(a.num_nodes[b], 0), T) : 0;
  const int nd = rr / g, hd = hk * g + (rr - nd * g);
  uint16_t* o = static_cast<uint16_t*>(a.out) + (((size_t)b * T + nd) * a.Hq + hd) * kD + 4 * c4;
  if (rr >= nn * g) {
    *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const int Rpad = row_tiles * kTileRows;
  const size_t bh = (size_t)b * a.Hkv + hk;
  const size_t nbh = (size_t)a.batch * a.Hkv;
  const size_t pbase = (bh * Rpad + rr) * kD + 4 * c4, pstride = nbh * Rpad * kD;
  const size_t mbase = (bh * Rpad + rr) * 2, mstride = nbh * Rpad * 2;
  // running merge over groups of kU splits (one group when nsplit <= kU)
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z0 = 0; z0 < nsplit; z0 += kU) {
    float2 ml[kU];
    float4 oz[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int zz = min(z0 + j, nsplit - 1);
      ml[j] = *reinterpret_cast<const float2*>(part_ml + mbase + zz * mstride);
      oz[j] = *reinterpret_cast<const float4*>(part_o + pbase + zz * pstride);
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (z0 + j < nsplit) Mg = fmaxf(Mg, ml[j].x);
    if (Mg == -INFINITY) continue;  // no key reached this row yet
    const float sc = __builtin_amdgcn_exp2f(M - Mg);  // rescale of the groups before
    den *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const float e = (z0 + j < nsplit) ? __builtin_amdgcn_exp2f(ml[j].x - Mg) : 0.f;
      den += e * ml[j].y;
      acc.x += e * oz[j].x;
      acc.y += e * oz[j].y;
      acc.z += e * oz[j].z;
      acc.w += e * oz[j].w;
    }
    M = Mg;
  }
  const float inv = den > 0.f ? 1.0f / den : 0.0f;
  floatx2 lo2 = {acc.x * inv, acc.y * inv}, hi2 = {acc.z * inv, acc.w * inv};
  bf16x2 l2 = __builtin_convertvector(lo2, bf16x2);
  bf16x2 h2 = __builtin_convertvector(hi2, bf16x2);
  bf16x4 o4 = {l2[0], l2[1], h2[0], h2[1]};
  *reinterpret_cast<bf16x4*>(o) = o4;
  const bool bad = !__builtin_isfinite(lo2[0]) | !__builtin_isfinite(lo2[1]) |
                   !__builtin_isfinite(hi2[0]) | !__builtin_isfinite(hi2[1]);
  if (bad) set_status(a.status, b, kStatusNonfinite);
}

// ------------------------------------------------------------------ fp32 path
// One thread per query row (b, i, h); fp32 online softmax over the allowed keys.
template <int D>
__global__ __launch_bounds__(128) void k_attn_simple(AttnArgs a) {
  const int64_t rid = (int64_t)blockIdx.x * 128 + threadIdx.x;
  const int64_t nrows = (int64_t)a.batch * a.T * a.Hq;
  if (rid >= nrows) return;
  const int h = (int)(rid % a.Hq);
  const int i = (int)((rid / a.Hq) % a.T);
  const int b = (int)(rid / ((int64_t)a.Hq * a.T));
  const float* Q = static_cast<const float*>(a.q);
  const float* Kg = static_cast<const float*>(a.k);
  const float* Vg = static_cast<const float*>(a.v);
  float* O = static_cast<float*>(a.out);
  const size_t obase = (((size_t)b * a.T + i) * a.Hq + h) * D;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  const bool kv_ok = kv_in_range(a.kv_offsets[b], a.prefix_lens[b], a.T, a.total_rows);
  const int nn = kv_ok ? min(max(a.num_nodes[b], 0), a.T) : 0;
  if (!kv_ok && i == 0 && h == 0) set_status(a.status, b, kStatusBadKv);
  float l = 0.0f;
  if (i < nn) {
    float q[D];
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = Q[obase + d];
    const int g = a.Hq / a.Hkv, hk = h / g;
    const int P = a.prefix_lens[b];
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
      const size_t kb = ((kv0 + j) * a.Hkv + hk) * D;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], Kg[kb + d], s);
      s *= c;
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vg[kb + d], acc[d] * alpha);
      m = mn;
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  bool bad = false;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float o = acc[d] * inv;
    bad |= !__builtin_isfinite(o);
    O[obase + d] = o;
  }
  if (bad) set_status(a.status, b, kStatusNonfinite);
}

// Clears the per-request status words before the attention kernels OR bits
// into them.
__global__ void k_zero_status(int32_t* status, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) status[i] = 0;
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

// Bytes of the fp16 V copy: vh_tiles key tiles per (request, kv-head).
size_t vh_bytes(int batch, int T, int Hkv, int max_prefix_len) {
  return (size_t)batch * Hkv * (size_t)vh_tiles(T, max_prefix_len) * kTileBytes;
}

// Split of each row tile's key range across workgroups: pick the count that
// minimises a simple time model -- rounds of resident workgroups (two per
// CU) times the key tiles per workgroup, plus the partial-result traffic of
// the merge -- with at least 4 key tiles per split.
AttnSplit plan_split(int dtype, int batch, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  AttnSplit s{1, 0, 1, 1, 0, 0, 0};
  if (dtype != 0 || D != kD) return s;
  const int g = Hq / Hkv;
  const int R = T * g;
  s.row_tiles = (int)(((long long)R + kTileRows - 1) / kTileRows);
  const long blocks = (long)batch * Hkv * s.row_tiles;
  const int tiles = (int)(((long long)max_prefix_len + kKeys - 1) / kKeys + (T + kKeys - 1) / kKeys);
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
  const long long nbh = (long long)batch * Hkv;
  s.chunk = nbh >= kXcds ? best : (int)std::max(1LL, best * nbh / kXcds);
  s.unit_chunks = (best + s.chunk - 1) / s.chunk;
  const long long units = nbh * s.unit_chunks;
  const long long per_unit8 = (units + kXcds - 1) / kXcds;
  // the grid, per_xcd * 8 workgroups, must fit in 31 bits; otherwise no plan
  if (per_unit8 > 0x7FFFFFFFLL / kXcds / s.chunk / s.row_tiles) {
    s.nsplit = 0;
    return s;
  }
  s.units = (int)units;
  s.per_xcd = (int)(per_unit8 * s.chunk * s.row_tiles);
  s.preconv = (s.row_tiles >= kPreconvMinRowTiles && batch <= 65535 && Hkv <= 65535 &&
               vh_bytes(batch, T, Hkv, max_prefix_len) <= kPreconvMaxBytes)
                  ? 1
                  : 0;
  return s;
}

hipError_t launch_simple(const AttnArgs& a, hipStream_t st) {
  const int64_t nrows = (int64_t)a.batch * a.T * a.Hq;
  dim3 grid((unsigned)((nrows + 127) / 128)), block(128);
  switch (a.D) {
    case 32: hipLaunchKernelGGL((k_attn_simple<32>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_attn_simple<64>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_attn_simple<128>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int dtype, int batch, int T, int Hq, int Hkv, int D,
                            int max_prefix_len) {
  const AttnSplit s = plan_split(dtype, batch, T, Hq, Hkv, D, max_prefix_len);
  if (s.nsplit == 0) return 0;  // no launchable grid for this shape
  size_t bytes = 0;
  if (s.nsplit > 1) {
    const size_t rows = (size_t)s.nsplit * batch * Hkv * s.row_tiles * kTileRows;
    bytes = align_up(rows * kD * 4, 256) + align_up(rows * 2 * 4, 256);
  }
  if (s.preconv) bytes += align_up(vh_bytes(batch, T, Hkv, max_prefix_len), 256);
  return bytes ? bytes : 256;
}

hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  if (a.status) {
    hipLaunchKernelGGL(k_zero_status, dim3((a.batch + 255) / 256), dim3(256), 0, st, a.status,
                       a.batch);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // f32 (any D); bf16 is D = 128 only (checked by the caller)
  if (a.dtype == 1) return launch_simple(a, st);
  const AttnSplit s = plan_split(a.dtype, a.batch, a.T, a.Hq, a.Hkv, a.D, a.max_prefix_len);
  if (s.nsplit == 0) return hipErrorInvalidConfiguration;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  char* p = static_cast<char*>(ws);
  if (s.nsplit > 1) {
    const size_t rows = (size_t)s.nsplit * a.batch * a.Hkv * s.row_tiles * kTileRows;
    part_o = reinterpret_cast<float*>(p);
    p += align_up(rows * kD * 4, 256);
    part_ml = reinterpret_cast<float*>(p);
    p += align_up(rows * 2 * 4, 256);
  }
  uint16_t* vh = nullptr;
  if (s.preconv) {
    vh = reinterpret_cast<uint16_t*>(p);
    hipLaunchKernelGGL(k_v_f16, dim3((unsigned)vh_tiles(a.T, a.max_prefix_len), a.Hkv, a.batch),
                       dim3(256), 0, st, a, vh);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(s.per_xcd * kXcds), block(256);
  hipLaunchKernelGGL(k_attn_mfma, grid, block, 0, st, a, s, part_o, part_ml, (const uint16_t*)vh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.nsplit <= 1) return e;
  const int R = a.T * (a.Hq / a.Hkv);
  dim3 cgrid((R + 7) / 8, a.batch * a.Hkv);
  hipLaunchKernelGGL(k_attn_combine, cgrid, block, 0, st, a, s.nsplit, s.row_tiles,
                     (const float*)part_o, (const float*)part_ml);
  return hipGetLastError();
}

}  // namespace ddt
