// Device-side helpers shared by the DDTree kernels (gfx950, wave64).
//
// Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees"
// (Ringel, Romano), summary page -- cited as [BDDT <section>].
//
// Compile with -ffp-contract=off: the per-position log-softmax must round
// exactly as specified below so that tree order (which compares sums of
// log-probabilities across depths) is reproducible to the bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddt {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Monotone map float -> uint32: a < b  <=>  ord(a) < ord(b) (no NaN input).
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_to_float(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(b);
}

// ---------------------------------------------------------------------------
// Per-position log-softmax arithmetic [BDDT §3, §4.3: log space keeps order].
//
// exp_fixed(d) = rint(2^44 * E(d)), E(d) ~ e^d for d <= 0:
//   t = fp32(d * fp32(log2 e)), clamped at -64; n = rint(t); f = t - n;
//   2^f by the degree-5 Taylor polynomial of 2^f, coefficients (ln 2)^k/k!
//   rounded to fp32, Horner with fused multiply-adds; scaled by 2^(n+44).
// Returned as a double holding an exact integer below 2^45, so that a
// thread's running sum stays exact (< 2^53) and the row sum is exact in
// uint64 regardless of summation order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double exp_fixed(float d) {
  float t = d * 0x1.715476p+0f;
  t = fmaxf(t, -64.0f);
  float n = rintf(t);
  float f = t - n;
  // The Horner steps run on the coefficients times 2^44: each step is then
  // exactly 2^44 times the unscaled one (scaling by a power of two commutes
  // with rounding while every value stays normal), which saves the + 44 on
  // the exponent.
  float p = 0x1.5d87fep+34f;            // (ln2)^5/120 * 2^44
  p = fmaf(p, f, 0x1.3b2ab6p+37f);      // (ln2)^4/24 * 2^44
  p = fmaf(p, f, 0x1.c6b08ep+39f);      // (ln2)^3/6 * 2^44
  p = fmaf(p, f, 0x1.ebfbe0p+41f);      // (ln2)^2/2 * 2^44
  p = fmaf(p, f, 0x1.62e430p+43f);      // ln2 * 2^44
  p = fmaf(p, f, 0x1p+44f);             // 1 * 2^44
  float e = ldexpf(p, (int)n);
  return (double)rintf(e);
}

// Natural log in fp64 for s >= 1: s = mant * 2^k, mant in [sqrt(1/2), sqrt(2)),
// ln s = k ln2 + 2 atanh(z), z = (mant-1)/(mant+1), atanh by its odd series
// through z^23 (Horner in z^2). Every step is one IEEE-754 double operation.
__device__ __forceinline__ double log_series(double s) {
  int k;
  double mant = frexp(s, &k);
  if (mant < 0x1.6a09e667f3bcdp-1) {
    mant = mant * 2.0;
    k = k - 1;
  }
  double z = (mant - 1.0) / (mant + 1.0);
  double w = z * z;
  double a = 1.0 / 23.0;
  a = a * w + 1.0 / 21.0;
  a = a * w + 1.0 / 19.0;
  a = a * w + 1.0 / 17.0;
  a = a * w + 1.0 / 15.0;
  a = a * w + 1.0 / 13.0;
  a = a * w + 1.0 / 11.0;
  a = a * w + 1.0 / 9.0;
  a = a * w + 1.0 / 7.0;
  a = a * w + 1.0 / 5.0;
  a = a * w + 1.0 / 3.0;
  a = a * w + 1.0;
  double head = (double)k * 0x1.62e42fefa39efp-1;
  double tail = (2.0 * z) * a;
  return head + tail;
}

// Fixed-point row sum S (units of 2^-44) to its log: fp32(ln(S * 2^-44)).
__device__ __forceinline__ float lse_from_fixed(uint64_t S) {
  double hi = (double)(uint32_t)(S >> 32) * 4294967296.0;
  double lo = (double)(uint32_t)(S & 0xffffffffu);
  return (float)log_series((hi + lo) * 0x1p-44);
}

// ---------------------------------------------------------------------------
// Wave-level helpers.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, kWave);
    v = w < v ? w : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave reductions through DPP row operations (no LDS round trip, unlike the
// shuffles above): lane ^ 1, lane ^ 2, the other quad of each 8, the other 8
// of each 16, then row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3).
// Lane 63 then holds the reduction over all 64 lanes; v_readlane returns it
// to every lane. Rows not written by a step keep `identity`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_src(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <class F>
__device__ __forceinline__ uint32_t dpp_reduce(uint32_t v, uint32_t identity, F op) {
  v = op(v, dpp_src<0xB1, 0xF>(identity, v));
  v = op(v, dpp_src<0x4E, 0xF>(identity, v));
  v = op(v, dpp_src<0x141, 0xF>(identity, v));
  v = op(v, dpp_src<0x140, 0xF>(identity, v));
  v = op(v, dpp_src<0x142, 0xA>(identity, v));
  v = op(v, dpp_src<0x143, 0xC>(identity, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_src64(uint64_t identity, uint64_t v) {
  const uint32_t lo = dpp_src<CTRL, ROW_MASK>((uint32_t)identity, (uint32_t)v);
  const uint32_t hi = dpp_src<CTRL, ROW_MASK>((uint32_t)(identity >> 32), (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <class F>
__device__ __forceinline__ uint64_t dpp_reduce64(uint64_t v, uint64_t identity, F op) {
  v = op(v, dpp_src64<0xB1, 0xF>(identity, v));
  v = op(v, dpp_src64<0x4E, 0xF>(identity, v));
  v = op(v, dpp_src64<0x141, 0xF>(identity, v));
  v = op(v, dpp_src64<0x140, 0xF>(identity, v));
  v = op(v, dpp_src64<0x142, 0xA>(identity, v));
  v = op(v, dpp_src64<0x143, 0xC>(identity, v));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  return __uint_as_float(dpp_reduce(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  return dpp_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_or_dpp(uint32_t v) {
  return dpp_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a | b; });
}
__device__ __forceinline__ uint64_t wave_sum_u64_dpp(uint64_t v) {
  return dpp_reduce64(v, 0ull, [](uint64_t a, uint64_t b) { return a + b; });
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  return dpp_reduce64(v, 0ull, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

// The k-th largest (k >= 1) of the 64 lanes' values, by a radix select on
// ballots, two bits per step: the largest t with at least k lanes holding
// >= t. Returns 0 when k > 64.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int k) {
  uint32_t t = 0;
#pragma unroll
  for (int sh = 30; sh >= 0; sh -= 2) {
    const uint32_t c1 = t | (1u << sh), c2 = t | (2u << sh), c3 = t | (3u << sh);
    const int n1 = __popcll(__ballot(v >= c1));
    const int n2 = __popcll(__ballot(v >= c2));
    const int n3 = __popcll(__ballot(v >= c3));
    t = n3 >= k ? c3 : (n2 >= k ? c2 : (n1 >= k ? c1 : t));
  }
  return t;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int w = __shfl_up(v, o, kWave);
    if (lane >= o) v += w;
  }
  return v;
}

}  // namespace ddt
