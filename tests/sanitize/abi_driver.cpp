// Host-side checks of the C ABI (include/ddtree.h) under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with arguments it
// must reject -- null pointers, sizes out of range, unsupported dtypes and
// shapes, missing or short workspaces, NaN and infinite scalars -- and each
// call must return its documented status without enqueuing anything. The
// workspace-size queries are called over extreme shapes (INT_MAX included):
// the planning arithmetic behind them must not overflow a signed integer.
//
// No call here passes validation, so no kernel is ever launched; the device
// pointers are stand-ins that host code never dereferences. The library
// sources are compiled for the host only, with the sanitizers (the test
// tests/test_sanitize_cpu.py builds and runs this).
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <climits>
#include <initializer_list>
#include <limits>

#include "ddtree.h"

static int g_fail = 0;

#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (call);                                                                \
    if (got_ != (want)) {                                                                   \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call,   \
              got_, (int)(want));                                                           \
      g_fail = 1;                                                                           \
    }                                                                                       \
  } while (0)

namespace {

// Stand-in device addresses: non-null, 256-byte aligned, never dereferenced.
template <typename T>
T* fake(uintptr_t slot) {
  return reinterpret_cast<T*>((uintptr_t)0x100000 + 0x1000 * slot);
}

const float kNaN = std::numeric_limits<float>::quiet_NaN();
const float kInf = std::numeric_limits<float>::infinity();

void build_calls() {
  const void* x = fake<void>(1);
  const int32_t* roots = fake<int32_t>(2);
  int32_t *tok = fake<int32_t>(3), *par = fake<int32_t>(4), *dep = fake<int32_t>(5);
  float* sc = fake<float>(6);
  int32_t* nn = fake<int32_t>(7);
  uint64_t* mask = fake<uint64_t>(8);
  int32_t* ttok = fake<int32_t>(9);
  float* tlp = fake<float>(10);
  int32_t* st = fake<int32_t>(11);
  void* ws = fake<void>(12);
  const size_t need = ddtree_build_workspace_size(4, 32, 151936, 16, 512);
  if (need == 0) {
    fprintf(stderr, "build workspace size of a valid shape is 0\n");
    g_fail = 1;
  }
  auto call = [&](const void* lg, int dt, const int32_t* r, int b, int L, int V, int K, int N,
                  float tau, int32_t* t, int32_t* p, int32_t* d, float* s, int32_t* n,
                  void* w, size_t wb) {
    return ddtree_build(lg, (ddtree_dtype)dt, r, b, L, V, K, N, tau, t, p, d, s, n, mask, ttok,
                        tlp, st, w, wb, nullptr);
  };
  const int A = DDTREE_ERR_ARG, U = DDTREE_ERR_UNSUPPORTED, W = DDTREE_ERR_WORKSPACE;
  EXPECT(call(nullptr, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, ws, need), A);
  EXPECT(call(x, 0, nullptr, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, ws, need), A);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, nullptr, par, dep, sc, nn, ws, need), A);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, nullptr, dep, sc, nn, ws, need), A);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, nullptr, sc, nn, ws, need), A);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, nullptr, nn, ws, need), A);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nullptr, ws, need), A);
  const int bad_sizes[][5] = {{0, 32, 151936, 16, 512}, {4, 0, 151936, 16, 512},
                              {4, 32, 0, 16, 512},      {4, 32, 151936, 0, 512},
                              {4, 32, 151936, 16, 0},   {-1, 32, 151936, 16, 512},
                              {4, 32, 8, 16, 512},      {INT_MIN, INT_MIN, INT_MIN, INT_MIN, 1}};
  for (const auto& s : bad_sizes)
    EXPECT(call(x, 0, roots, s[0], s[1], s[2], s[3], s[4], 1, tok, par, dep, sc, nn, ws, need),
           A);
  for (float tau : {-1.0f, kNaN, kInf, -kInf})
    EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, tau, tok, par, dep, sc, nn, ws, need), A);
  for (int dt : {2, -1, 7})
    EXPECT(call(x, dt, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, ws, need), U);
  const int big[][5] = {{4, DDTREE_MAX_L + 1, 1000, 4, 8},  {4, 4, 1000, DDTREE_MAX_K + 1, 8},
                        {4, 4, 1000, 4, DDTREE_MAX_N + 1},  {4, 4, DDTREE_MAX_V + 1, 4, 8},
                        {INT_MAX, 2, 1000, 4, 8},           {INT_MAX, INT_MAX, INT_MAX, 4, 8}};
  for (const auto& s : big)
    EXPECT(call(x, 0, roots, s[0], s[1], s[2], s[3], s[4], 1, tok, par, dep, sc, nn, ws, need),
           U);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, nullptr, need), W);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, ws, need - 1), W);
  EXPECT(call(x, 0, roots, 4, 32, 151936, 16, 512, 1, tok, par, dep, sc, nn, ws, 0), W);
  // the variant without a workspace: same checks, then the static scratch limit
  EXPECT(ddtree_build_noalloc(nullptr, DDTREE_BF16, roots, 4, 32, 151936, 16, 512, 1, tok, par,
                              dep, sc, nn, mask, ttok, tlp, st, nullptr),
         A);
  EXPECT(ddtree_build_noalloc(x, (ddtree_dtype)3, roots, 4, 32, 151936, 16, 512, 1, tok, par,
                              dep, sc, nn, mask, ttok, tlp, st, nullptr),
         U);
  EXPECT(ddtree_build_noalloc(x, DDTREE_BF16, roots, 4096, 32, 151936, 16, 512, 1, tok, par,
                              dep, sc, nn, mask, ttok, tlp, st, nullptr),
         DDTREE_ERR_SCRATCH);
}

void mask_calls() {
  const int32_t *p = fake<int32_t>(1), *n = fake<int32_t>(2);
  uint64_t* m = fake<uint64_t>(3);
  EXPECT(ddtree_mask(nullptr, n, 4, 65, m, nullptr), DDTREE_ERR_ARG);
  EXPECT(ddtree_mask(p, nullptr, 4, 65, m, nullptr), DDTREE_ERR_ARG);
  EXPECT(ddtree_mask(p, n, 4, 65, nullptr, nullptr), DDTREE_ERR_ARG);
  EXPECT(ddtree_mask(p, n, 0, 65, m, nullptr), DDTREE_ERR_ARG);
  EXPECT(ddtree_mask(p, n, 4, 0, m, nullptr), DDTREE_ERR_ARG);
  EXPECT(ddtree_mask(p, n, 4, DDTREE_MAX_N + 2, m, nullptr), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_mask(p, n, INT_MIN, INT_MIN, m, nullptr), DDTREE_ERR_ARG);
}

void verify_calls() {
  const void *q = fake<void>(1), *k = fake<void>(2), *v = fake<void>(3);
  const int64_t* offs = fake<int64_t>(4);
  const int32_t *P = fake<int32_t>(5), *nn = fake<int32_t>(6);
  const uint64_t* m = fake<uint64_t>(7);
  void* out = fake<void>(8);
  int32_t* st = fake<int32_t>(9);
  void* ws = fake<void>(10);
  const size_t need = ddtree_verify_workspace_size(DDTREE_BF16, 4, 513, 64, 8, 128, 65536);
  auto call = [&](const void* qq, int dt, int b, int T, int Hq, int Hkv, int D, int maxp,
                  int64_t rows, float scale, void* o, void* w, size_t wb) {
    return ddtree_verify_attn(qq, k, v, (ddtree_dtype)dt, offs, P, nn, m, b, T, Hq, Hkv, D, maxp,
                              rows, scale, o, st, w, wb, nullptr);
  };
  const int A = DDTREE_ERR_ARG, U = DDTREE_ERR_UNSUPPORTED, W = DDTREE_ERR_WORKSPACE;
  const int64_t R = 4 * (65536 + 513);
  EXPECT(call(nullptr, 0, 4, 513, 64, 8, 128, 65536, R, 0, out, ws, need), A);
  EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, R, 0, nullptr, ws, need), A);
  EXPECT(ddtree_verify_attn(q, nullptr, v, DDTREE_BF16, offs, P, nn, m, 4, 513, 64, 8, 128, 65536,
                            R, 0, out, st, ws, need, nullptr),
         A);
  EXPECT(ddtree_verify_attn(q, k, v, DDTREE_BF16, offs, P, nn, nullptr, 4, 513, 64, 8, 128,
                            65536, R, 0, out, st, ws, need, nullptr),
         A);
  const int bad[][6] = {{0, 513, 64, 8, 128, 65536}, {4, 0, 64, 8, 128, 65536},
                        {4, 513, 0, 8, 128, 65536},  {4, 513, 64, 0, 128, 65536},
                        {4, 513, 64, 8, 0, 65536},   {4, 513, 64, 8, 128, -1},
                        {4, 513, 64, 7, 128, 65536}, {INT_MIN, 1, 1, 1, 1, INT_MIN}};
  for (const auto& s : bad)
    EXPECT(call(q, 0, s[0], s[1], s[2], s[3], s[4], s[5], R, 0, out, ws, need), A);
  EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, 0, 0, out, ws, need), A);
  EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, -5, 0, out, ws, need), A);
  for (float s : {kNaN, kInf, -kInf})
    EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, R, s, out, ws, need), A);
  EXPECT(call(q, 5, 4, 513, 64, 8, 128, 65536, R, 0, out, ws, need), U);
  EXPECT(call(q, 0, 4, DDTREE_MAX_N + 2, 64, 8, 128, 65536, R, 0, out, ws, need), U);
  EXPECT(call(q, 0, 4, 513, 64, 8, 96, 65536, R, 0, out, ws, need), U);
  EXPECT(call(q, 0, 4, 513, 64, 8, 64, 65536, R, 0, out, ws, need), U);  // bf16 is D = 128 only
  EXPECT(call(q, 1, 4, 513, 64, 8, 256, 65536, R, 0, out, ws, need), U);
  EXPECT(call(q, 0, INT_MAX, 1025, 64, 8, 128, 65536, R, 0, out, ws, need), U);
  EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, R, 0, out, nullptr, need), W);
  EXPECT(call(q, 0, 4, 513, 64, 8, 128, 65536, R, 0, out, ws, need - 1), W);
}

void accept_calls() {
  const void* tl = fake<void>(1);
  const int32_t *ids = fake<int32_t>(2), *tok = fake<int32_t>(3), *par = fake<int32_t>(4);
  const int32_t* nn = fake<int32_t>(5);
  int32_t *acc = fake<int32_t>(6), *accn = fake<int32_t>(7), *alen = fake<int32_t>(8);
  int32_t *bonus = fake<int32_t>(9), *tgt = fake<int32_t>(10);
  void* ws = fake<void>(11);
  const size_t need = ddtree_accept_workspace_size(4, 513);
  const int A = DDTREE_ERR_ARG, U = DDTREE_ERR_UNSUPPORTED, W = DDTREE_ERR_WORKSPACE;
  auto call = [&](const void* lg, const int32_t* id, int dt, int b, int T, int V, int L,
                  int32_t* ac, void* w, size_t wb) {
    return ddtree_accept(lg, (ddtree_dtype)dt, id, tok, par, nn, b, T, V, L, ac, accn, alen,
                         bonus, tgt, w, wb, nullptr);
  };
  EXPECT(call(nullptr, nullptr, 0, 4, 513, 151936, 32, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 0, 4, 513, 151936, 32, nullptr, ws, need), A);
  EXPECT(call(tl, nullptr, 0, 0, 513, 151936, 32, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 0, 4, 0, 151936, 32, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 0, 4, 513, 151936, 0, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 0, 4, 513, 0, 32, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 0, INT_MIN, INT_MIN, INT_MIN, INT_MIN, acc, ws, need), A);
  EXPECT(call(tl, nullptr, 4, 4, 513, 151936, 32, acc, ws, need), U);
  EXPECT(call(tl, nullptr, 0, 4, DDTREE_MAX_N + 2, 151936, 32, acc, ws, need), U);
  EXPECT(call(tl, nullptr, 0, 4, 513, 151936, DDTREE_MAX_L + 1, acc, ws, need), U);
  EXPECT(call(tl, nullptr, 0, INT_MAX, 1025, 151936, 32, acc, ws, need), U);
  EXPECT(call(tl, nullptr, 0, 4, 513, 151936, 32, acc, nullptr, need), W);
  EXPECT(call(nullptr, ids, 0, 4, 513, 0, 32, acc, ws, need - 1), W);
  // sampled acceptance
  auto samp = [&](const void* lg, int dt, int b, int T, int V, int L, float temp, int32_t* tt,
                  void* w, size_t wb) {
    return ddtree_accept_sample(lg, (ddtree_dtype)dt, tok, par, nn, b, T, V, L, temp, 1, 2, acc,
                                accn, alen, bonus, tt, w, wb, nullptr);
  };
  EXPECT(samp(nullptr, 0, 4, 513, 151936, 32, 1, tgt, ws, need), A);
  for (float t : {0.0f, -1.0f, kNaN, kInf})
    EXPECT(samp(tl, 0, 4, 513, 151936, 32, t, tgt, ws, need), A);
  EXPECT(samp(tl, 0, 4, 513, 0, 32, 1, tgt, ws, need), A);
  EXPECT(samp(tl, 9, 4, 513, 151936, 32, 1, tgt, ws, need), U);
  EXPECT(samp(tl, 0, 4, 513, DDTREE_MAX_V + 1, 32, 1, tgt, ws, need), U);
  EXPECT(samp(tl, 0, 4, 513, INT_MAX, 32, 1, tgt, ws, need), U);
  EXPECT(samp(tl, 0, INT_MAX, 1025, 1000, 32, 1, tgt, ws, need), U);
  EXPECT(samp(tl, 0, 4, 513, 151936, 32, 1, nullptr, nullptr, need), W);
  EXPECT(samp(tl, 0, 4, 513, 151936, 32, 1, nullptr, ws, need - 1), W);
}

void commit_calls() {
  void *k = fake<void>(1), *v = fake<void>(2);
  const int64_t* offs = fake<int64_t>(3);
  const int32_t *P = fake<int32_t>(4), *alen = fake<int32_t>(5), *an = fake<int32_t>(6);
  const int32_t* bonus = fake<int32_t>(7);
  int32_t *np = fake<int32_t>(8), *nr = fake<int32_t>(9);
  const int A = DDTREE_ERR_ARG, U = DDTREE_ERR_UNSUPPORTED;
  auto call = [&](void* kk, int dt, int b, int Hkv, int D, int L, int T, int64_t rows,
                  int32_t* newp, const int32_t* pl) {
    return ddtree_commit_kv(kk, v, (ddtree_dtype)dt, offs, pl, alen, an, bonus, b, Hkv, D, L, T,
                            rows, newp, nr, nullptr);
  };
  EXPECT(call(nullptr, 0, 4, 8, 128, 32, 513, 1 << 20, np, P), A);
  EXPECT(call(k, 0, 4, 8, 128, 32, 513, 1 << 20, nullptr, P), A);
  EXPECT(call(k, 0, 4, 8, 128, 32, 513, 1 << 20, np, nullptr), A);
  EXPECT(call(k, 0, 4, 8, 128, 32, 513, 1 << 20, np, np), A);  // output aliases the input
  EXPECT(call(k, 0, 0, 8, 128, 32, 513, 1 << 20, np, P), A);
  EXPECT(call(k, 0, 4, 8, 128, 32, 513, 0, np, P), A);
  EXPECT(call(k, 0, INT_MIN, INT_MIN, INT_MIN, INT_MIN, INT_MIN, INT64_MIN, np, P), A);
  EXPECT(call(k, 6, 4, 8, 128, 32, 513, 1 << 20, np, P), U);
  EXPECT(call(k, 0, 4, 8, 128, DDTREE_MAX_L + 1, 513, 1 << 20, np, P), U);
  EXPECT(call(k, 0, 4, 8, 128, 32, DDTREE_MAX_N + 2, 1 << 20, np, P), U);
  EXPECT(call(k, 0, 4, 65536, 128, 32, 513, 1 << 20, np, P), U);
  EXPECT(call(k, 0, 4, 8, 4, 32, 513, 1 << 20, np, P), U);     // 8-byte rows
  EXPECT(call(k, 1, 4, 8, 512, 32, 513, 1 << 20, np, P), U);   // 2 KB rows
  EXPECT(call(k, 0, 4, 8, INT_MAX, 32, 513, 1 << 20, np, P), U);
  EXPECT(call(reinterpret_cast<char*>(k) + 8, 0, 4, 8, 128, 32, 513, 1 << 20, np, P), U);
}

void size_queries() {
  const int vals[] = {INT_MIN, -1, 0, 1, 2, 63, 64, 65, 1000, 151936, DDTREE_MAX_V, 1 << 24,
                      INT_MAX};
  size_t sink = 0;
  for (int b : vals)
    for (int L : {1, 16, DDTREE_MAX_L, INT_MAX})
      for (int V : vals)
        for (int K : {1, 8, DDTREE_MAX_K, DDTREE_MAX_K + 1}) {
          const size_t s = ddtree_build_workspace_size(b, L, V, K, 512);
          if ((b < 1 || V < 1) && s != 0) {
            fprintf(stderr, "build workspace %d %d %d %d: %zu, expected 0\n", b, L, V, K, s);
            g_fail = 1;
          }
          sink += s;
        }
  for (int dt : {0, 1, 3})
    for (int b : vals)
      for (int T : {INT_MIN, 0, 1, 65, 513, 1025, DDTREE_MAX_N + 1, INT_MAX})
        for (int hq : {1, 8, 64, INT_MAX})
          for (int D : {32, 128})
            for (int maxp : {INT_MIN, 0, 1, 65536, INT_MAX}) {
              const size_t s = ddtree_verify_workspace_size((ddtree_dtype)dt, b, T, hq, 1, D, maxp);
              if ((b < 1 || T < 1 || maxp < 0) && s != 0) {
                fprintf(stderr, "verify workspace %d %d %d: %zu, expected 0\n", b, T, maxp, s);
                g_fail = 1;
              }
              sink += s;
            }
  for (int b : vals)
    for (int T : {INT_MIN, 0, 1, 65, 1025, INT_MAX}) {
      const size_t s = ddtree_accept_workspace_size(b, T);
      if ((b < 1 || T < 1) && s != 0) {
        fprintf(stderr, "accept workspace %d %d: %zu, expected 0\n", b, T, s);
        g_fail = 1;
      }
      sink += s;
    }
  printf("size queries done (%zu)\n", sink % 997);
}

}  // namespace

int main() {
  if (ddtree_version() != DDTREE_VERSION) g_fail = 1;
  for (int s = -12; s <= 12; ++s)
    if (!ddtree_strerror(s)) g_fail = 1;
  size_queries();
  build_calls();
  mask_calls();
  verify_calls();
  accept_calls();
  commit_calls();
  if (g_fail) return 1;
  printf("abi driver: every rejected call returned its status\n");
  return 0;
}
