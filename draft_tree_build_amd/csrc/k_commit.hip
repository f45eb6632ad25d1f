// KV compaction of the accepted path and the bonus hand-off on gfx950.
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page, §4.1: the matched path is accepted and the
// first unmatched target token becomes the bonus token, the root of the next
// round. The verify wrote the tree's K/V rows after each request's prefix in
// node order (node i at row P + i); committing the accepted nodes
// a_0 .. a_{n-1} moves their rows to P + 1 .. P + n (the root, node 0, is
// already at row P), the new prefix length is P + 1 + n and the bonus is the
// next root. All moves read the rows as they were before the first one.
//
// k_commit: one workgroup per (request, kv-head, K or V). The head's slice of
// every moved row (D * esize bytes, 16-byte chunks) is read into registers,
// the workgroup meets at a barrier, and only then are the slices written:
// slices of other heads and of the other tensor are disjoint, so the moves
// are the simultaneous assignment above whatever their order. Rows already
// in place (a_k == k + 1) are not rewritten. Each workgroup checks the
// request's inputs itself; a malformed request is left untouched and gets
// -1 as new prefix length and next root.
#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

constexpr int kCommitBlock = 256;
constexpr int kCommitPer = 16;  // chunks per thread: 64 rows x 64 chunks / 256 threads

__global__ __launch_bounds__(kCommitBlock) void k_commit(CommitArgs a) {
  __shared__ int s_ok, s_n;
  __shared__ int64_t s_row0;
  __shared__ int32_t s_src[64];
  const int b = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const int tid = threadIdx.x;
  if (tid < 64) {  // wave 0 validates the request
    // every input of the request is requested in one round trip
    int32_t bonus = a.bonus[b];
    const int n = a.accept_len[b];
    const int64_t off = a.kv_offsets[b];
    const int64_t P = a.prefix_lens[b];
    const int32_t listed = tid < a.L ? a.accepted_nodes[(size_t)b * a.L + tid] : 0;
    asm volatile("" : "+v"(bonus));  // keeps the load beside the others
    bool ok = n >= 0 && n <= a.L && n <= a.T - 1 && off >= 0 && P >= 0 &&
              off + P + a.T <= a.total_rows;
    const int src = (ok && tid < n) ? listed : 0;
    const bool bad = ok && tid < n && (src < 1 || src >= a.T);
    ok = ok && __ballot(bad) == 0;
    s_src[tid] = src;
    if (tid == 0) {
      s_ok = ok;
      s_n = n;
      s_row0 = off + P;
      if (h == 0 && which == 0) {
        a.new_prefix_lens[b] = ok ? (int32_t)(P + 1 + n) : -1;
        if (a.next_roots) a.next_roots[b] = ok ? bonus : -1;
      }
    }
  }
  __syncthreads();
  const int n = s_n;
  if (!s_ok || n == 0) return;
  const int cpr = a.cpr;
  const int total = n * cpr;
  const int64_t row0 = s_row0;
  uint4* base = static_cast<uint4*>(which ? a.v_cache : a.k_cache);
  // chunk c of head h in row r of the region: ((row0 + r) * Hkv + h) * cpr + c
  int kq[kCommitPer], srcq[kCommitPer];
#pragma unroll
  for (int q = 0; q < kCommitPer; ++q) {
    const int id = tid + q * kCommitBlock;
    kq[q] = id < total ? id / cpr : -1;
    srcq[q] = s_src[kq[q] < 0 ? 0 : kq[q]];
  }
  // all source indices are in registers before the first load is formed
#pragma unroll
  for (int q = 0; q < kCommitPer; ++q) asm volatile("" : "+v"(srcq[q]));
  uint4 val[kCommitPer];
#pragma unroll
  for (int q = 0; q < kCommitPer; ++q) {
    const int id = tid + q * kCommitBlock;
    const int c = kq[q] < 0 ? 0 : id - kq[q] * cpr;
    val[q] = base[((row0 + srcq[q]) * a.Hkv + h) * cpr + c];
  }
  // every value has arrived before any thread passes the barrier
#pragma unroll
  for (int q = 0; q < kCommitPer; ++q)
    asm volatile("" : "+v"(val[q].x), "+v"(val[q].y), "+v"(val[q].z), "+v"(val[q].w));
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kCommitPer; ++q) {
    const int k = kq[q];
    if (k >= 0 && srcq[q] != k + 1) {  // rows already in place are not rewritten
      const int id = tid + q * kCommitBlock;
      base[((row0 + 1 + k) * a.Hkv + h) * cpr + (id - k * cpr)] = val[q];
    }
  }
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_commit, dim3(a.batch, a.Hkv, 2), dim3(kCommitBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace ddt
