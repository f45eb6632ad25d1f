// Calibration kernels for the measured peaks that the benchmark reports next
// to the published ones (a dense bf16 MFMA loop and an HBM read stream). They
// are not part of a DDTree round; nothing in the round calls them.
#include "ddtree_device.h"
#include "ddtree_internal.h"

namespace ddt {
namespace {

// Four independent accumulation chains of v_mfma_f32_32x32x16_bf16 per wave,
// enough to keep the matrix pipe issuing back to back (one chain alone waits
// on its own accumulator). Operands stay in registers: no memory traffic but
// one store per lane at the end, which keeps the loop from being removed.
__global__ __launch_bounds__(256) void k_probe_mfma(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.125f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.0625f * (float)(i + 1));
  }
  floatx16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Streaming read of nvec 16-byte vectors, grid-strided; each thread has
// eight loads in flight before it uses any. One word per workgroup written.
__global__ __launch_bounds__(256) void k_probe_read(const uint4* src, int64_t nvec, uint32_t* out) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base < nvec; base += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[min(base + j * stride, nvec - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  x = wave_or_dpp(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

hipError_t launch_probe_mfma(float* out, int grid, int iters, hipStream_t st) {
  hipLaunchKernelGGL(k_probe_mfma, dim3(grid), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(src),
                     bytes / 16, out);
  return hipGetLastError();
}

}  // namespace ddt
