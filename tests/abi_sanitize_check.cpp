// Host-only check of the C ABI's argument validation (abi.cpp), built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize_cpu.py.  The kernel launchers are replaced by the stubs
// below, which only record that a launch was requested, so every entry point
// runs its full validation on the host with fake device addresses: valid calls
// must reach exactly one launcher, invalid ones none, and no size arithmetic
// may overflow (UBSan aborts the run on any signed overflow, shift or
// out-of-range conversion; ASan on any bad memory access).
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "kernels.hpp"
#include "linattn.h"

// ----------------------------------------------------------------- launcher stubs
static int g_launches = 0;
static long long g_last_bh = -1, g_last_n = -1;

static hipError_t record(int BH, long long N) {
  ++g_launches;
  g_last_bh = BH;
  g_last_n = N;
  return hipSuccess;
}

namespace la {
int causal_block_tokens(int, int) { return 256; }
// Sizes of the same order as the real ones; the validation only compares them.
size_t causal_ws_bytes(int BH, int N, int D, int M, int) {
  return (size_t)BH * (size_t)((N + 255) / 256) * (size_t)(D * M + D) * 4;
}
size_t noncausal_ws_bytes(int BH, int, int D, int M, int) { return (size_t)(BH + 1) * (size_t)(D * M + D) * 4; }
size_t causal_bwd_ws_bytes(int BH, int N, int D, int M) { return (size_t)BH * (size_t)N * (size_t)(M + 2) * 4 + D; }
size_t deltanet_ws_bytes(int BH, int N, int D, int M) {
  return (size_t)BH * (size_t)((N + 63) / 64) * (size_t)(6 * D * M) * 4;
}
int featmap_dim(int map, int D) { return map == 4 ? D * D : 2 * map * D; }
size_t featmap_ws_bytes(int map, int BH, int N, int D, int M) {
  return (size_t)BH * (size_t)((N + 63) / 64) * (size_t)(featmap_dim(map, D) * (M + 1)) * 4;
}
hipError_t launch_causal(const void*, const void*, const void*, void*, int BH, int N, int, int, int, const float*,
                         const float*, float*, float*, void*, hipStream_t) {
  return record(BH, N);
}
hipError_t launch_noncausal(const void*, const void*, const void*, void*, int BH, int N, int, int, int, void*,
                            hipStream_t) {
  return record(BH, N);
}
hipError_t launch_causal_bwd(const void*, const void*, const void*, const void*, void*, void*, void*, int BH, int N,
                             int, int, int, void*, hipStream_t) {
  return record(BH, N);
}
hipError_t launch_decode(const void*, const void*, const void*, void*, float*, float*, int BH, int, int, int,
                         hipStream_t) {
  return record(BH, 1);
}
hipError_t launch_softmax_decode(const void*, const void*, const void*, void*, void*, void*, int BH, int L, int, int,
                                 int, int, hipStream_t) {
  return record(BH, L);
}
hipError_t launch_featmap(int, const void*, const void*, const void*, void*, int BH, int N, int, int, int, int,
                          const float*, const float*, float*, float*, void*, hipStream_t) {
  return record(BH, N);
}
hipError_t launch_deltanet(const void*, const void*, const void*, const void*, void*, int BH, int N, int, int, int,
                           const float*, float*, void*, hipStream_t) {
  return record(BH, N);
}
hipError_t launch_deltanet_step(const void*, const void*, const void*, const void*, void*, float*, int BH, int, int,
                                int, hipStream_t) {
  return record(BH, 1);
}
void* noalloc_scratch() { return (void*)(uintptr_t)((uint64_t)63 << 36); }
}  // namespace la

// ----------------------------------------------------------------- cases
static int g_fail = 0;

// Fake device addresses: 16-byte aligned and 2^36 apart, so no two overlap.
static void* P(int i) { return (void*)(uintptr_t)((uint64_t)(i + 1) << 36); }
static float* F(int i) { return (float*)P(i); }
static const size_t BIG = (size_t)1 << 40;

static void expect(const char* what, int got, int want, int launched_want) {
  const int before = g_launches;
  (void)before;
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, want %d\n", what, got, want);
    ++g_fail;
  }
  if (launched_want >= 0 && g_launches != launched_want) {
    fprintf(stderr, "FAIL %s: %d launches, want %d\n", what, g_launches, launched_want);
    ++g_fail;
  }
}

#define CHECK(what, call, want)                     \
  do {                                              \
    const int n0 = g_launches;                      \
    const int st = (call);                          \
    expect(what, st, want, n0 + ((want) == 0 ? 1 : 0)); \
  } while (0)
#define CHECK_NOLAUNCH(what, call, want)            \
  do {                                              \
    const int n0 = g_launches;                      \
    const int st = (call);                          \
    expect(what, st, want, n0);                     \
  } while (0)

static int causal(int B, int H, int N, int D, int M, int dt, void* o = P(3), void* q = P(0), size_t wsb = BIG,
                  const float* S0 = nullptr, const float* z0 = nullptr, float* So = nullptr, float* zo = nullptr) {
  return linattn_causal_fwd(q, P(1), P(2), o, B, H, N, D, M, dt, S0, z0, So, zo, P(9), wsb, nullptr);
}

int main() {
  // ---- causal
  CHECK("causal ok", causal(2, 16, 32768, 64, 64, 1), LINATTN_OK);
  if (g_last_bh != 32 || g_last_n != 32768) {
    fprintf(stderr, "FAIL causal launch args %lld %lld\n", g_last_bh, g_last_n);
    ++g_fail;
  }
  CHECK("causal state in place", causal(1, 8, 4096, 64, 32, 0, P(3), P(0), BIG, F(4), F(5), F(4), F(5)), LINATTN_OK);
  CHECK_NOLAUNCH("causal dtype", causal(1, 1, 16, 64, 64, 2), LINATTN_ERR_DTYPE);
  CHECK_NOLAUNCH("causal dtype neg", causal(1, 1, 16, 64, 64, -1), LINATTN_ERR_DTYPE);
  CHECK_NOLAUNCH("causal D", causal(1, 1, 16, 48, 64, 0), LINATTN_ERR_UNSUPPORTED);
  CHECK_NOLAUNCH("causal B<0", causal(-1, 1, 16, 64, 64, 0), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal N<0", causal(1, 1, INT_MIN, 64, 64, 0), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal D<0", causal(1, 1, 16, INT_MIN, 64, 0), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal BH huge", causal(INT_MAX, INT_MAX, 16, 64, 64, 0), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal rows huge", causal(1 << 15, 1 << 15, INT_MAX, 64, 64, 1), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal N huge", causal(1, 1, INT_MAX, 64, 64, 1), LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("causal null q", causal(1, 1, 16, 64, 64, 0, P(3), nullptr), LINATTN_ERR_NULL);
  CHECK_NOLAUNCH("causal misaligned", causal(1, 1, 16, 64, 64, 0, (char*)P(3) + 8), LINATTN_ERR_ALIGN);
  CHECK_NOLAUNCH("causal o aliases q", causal(1, 1, 16, 64, 64, 0, P(0)), LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("causal workspace", causal(1, 2, 4096, 64, 64, 1, P(3), P(0), 16), LINATTN_ERR_WORKSPACE);
  CHECK_NOLAUNCH("causal half state", causal(1, 1, 16, 64, 64, 0, P(3), P(0), BIG, F(4), nullptr), LINATTN_ERR_NULL);
  CHECK_NOLAUNCH("causal partial overlap",
                 causal(1, 1, 16, 64, 64, 0, P(3), P(0), BIG, F(4), F(5), F(4) + 4, F(5)), LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("causal empty", causal(0, 4, 16, 64, 64, 0), LINATTN_OK);
  CHECK_NOLAUNCH("causal N=0 no state", causal(2, 4, 0, 64, 64, 0), LINATTN_OK);
  CHECK("causal N=0 state", causal(2, 4, 0, 64, 64, 0, P(3), P(0), BIG, nullptr, nullptr, F(6), F(7)), LINATTN_OK);
  for (int B : {0, 1, 3, 1 << 10, 1 << 20, INT_MAX})
    for (int N : {0, 1, 255, 256, 1 << 20, INT_MAX}) {
      (void)linattn_causal_workspace_bytes(B, 16, N, 64, 64, 1);
      (void)linattn_noncausal_workspace_bytes(B, 16, N, 64, 64, 0);
      (void)linattn_causal_bwd_workspace_bytes(B, 16, N, 32, 64, 1);
      (void)deltanet_workspace_bytes(B, 16, N, 64, 32, 0);
      (void)linattn_fmap_workspace_bytes(B, 16, N, 64, 64, 0, LINATTN_FMAP_POLY2, 0);
    }

  // ---- non-causal
  CHECK("noncausal ok", linattn_noncausal_fwd(P(0), P(1), P(2), P(3), 2, 16, 32768, 64, 64, 1, P(9), BIG, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("noncausal no ws",
                 linattn_noncausal_fwd(P(0), P(1), P(2), P(3), 2, 16, 4096, 64, 64, 1, nullptr, 0, nullptr),
                 LINATTN_ERR_WORKSPACE);
  CHECK_NOLAUNCH("noncausal o aliases v",
                 linattn_noncausal_fwd(P(0), P(1), P(2), P(2), 2, 16, 4096, 64, 64, 1, P(9), BIG, nullptr),
                 LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("noncausal ws aliases q",
                 linattn_noncausal_fwd(P(0), P(1), P(2), P(3), 2, 16, 4096, 64, 64, 1, P(0), BIG, nullptr),
                 LINATTN_ERR_ALIAS);

  // ---- non-causal without allocation (static scratch)
  CHECK("noncausal noalloc ok", linattn_noncausal_fwd_noalloc(P(0), P(1), P(2), P(3), 2, 16, 32768, 64, 64, 1, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("noncausal noalloc too big",
                 linattn_noncausal_fwd_noalloc(P(0), P(1), P(2), P(3), 64, 64, 4096, 64, 64, 1, nullptr),
                 LINATTN_ERR_WORKSPACE);
  CHECK_NOLAUNCH("noncausal noalloc alias",
                 linattn_noncausal_fwd_noalloc(P(0), P(1), P(2), P(1), 2, 16, 4096, 64, 64, 1, nullptr),
                 LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("noncausal noalloc null", linattn_noncausal_fwd_noalloc(P(0), nullptr, P(2), P(3), 2, 16, 4096, 64,
                                                                         64, 1, nullptr),
                 LINATTN_ERR_NULL);
  CHECK_NOLAUNCH("noncausal noalloc empty", linattn_noncausal_fwd_noalloc(nullptr, nullptr, nullptr, nullptr, 2, 16,
                                                                          0, 64, 64, 1, nullptr),
                 LINATTN_OK);

  // ---- backward
  CHECK("bwd ok", linattn_causal_bwd(P(0), P(1), P(2), P(3), P(4), P(5), P(6), 2, 16, 32768, 64, 64, 1, P(9), BIG,
                                     nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("bwd dq aliases dk", linattn_causal_bwd(P(0), P(1), P(2), P(3), P(4), P(4), P(6), 1, 1, 64, 64, 64,
                                                         0, P(9), BIG, nullptr),
                 LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("bwd null dO", linattn_causal_bwd(P(0), P(1), P(2), nullptr, P(4), P(5), P(6), 1, 1, 64, 64, 64, 0,
                                                   P(9), BIG, nullptr),
                 LINATTN_ERR_NULL);

  // ---- decode step
  CHECK("decode ok", linattn_decode_step(P(0), P(1), P(2), P(3), F(4), F(5), 256, 16, 64, 64, 1, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("decode S aliases z",
                 linattn_decode_step(P(0), P(1), P(2), P(3), F(4), F(4), 256, 16, 64, 64, 1, nullptr),
                 LINATTN_ERR_ALIAS);
  CHECK_NOLAUNCH("decode huge", linattn_decode_step(P(0), P(1), P(2), P(3), F(4), F(5), INT_MAX, INT_MAX, 64, 64, 1,
                                                    nullptr),
                 LINATTN_ERR_SHAPE);

  // ---- softmax decode step
  CHECK("softmax ok", softmax_decode_step(P(0), P(1), P(2), P(3), P(4), P(5), 256, 16, 100, 1536, 64, 64, 1, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("softmax L out of range",
                 softmax_decode_step(P(0), P(1), P(2), P(3), P(4), P(5), 2, 2, 1536, 1536, 64, 64, 1, nullptr),
                 LINATTN_ERR_SHAPE);
  CHECK_NOLAUNCH("softmax L negative",
                 softmax_decode_step(P(0), P(1), P(2), P(3), P(4), P(5), 2, 2, INT_MIN, 1536, 64, 64, 1, nullptr),
                 LINATTN_ERR_SHAPE);

  // ---- feature maps
  CHECK("fmap ok", linattn_fmap_fwd(P(0), P(1), P(2), P(3), 4, 8, 4096, 64, 64, 0, LINATTN_FMAP_POLY2, 0, 1, nullptr,
                                    nullptr, F(6), F(7), P(9), BIG, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("fmap bad nu", linattn_fmap_fwd(P(0), P(1), P(2), P(3), 4, 8, 4096, 64, 64, 0, LINATTN_FMAP_DPFP, 4,
                                                 1, nullptr, nullptr, nullptr, nullptr, P(9), BIG, nullptr),
                 LINATTN_ERR_UNSUPPORTED);
  CHECK_NOLAUNCH("fmap noncausal with S0",
                 linattn_fmap_fwd(P(0), P(1), P(2), P(3), 4, 8, 4096, 64, 64, 0, LINATTN_FMAP_DPFP, 1, 0, F(4), F(5),
                                  nullptr, nullptr, P(9), BIG, nullptr),
                 LINATTN_ERR_UNSUPPORTED);
  CHECK_NOLAUNCH("fmap huge", linattn_fmap_fwd(P(0), P(1), P(2), P(3), 1 << 14, 1 << 14, INT_MAX, 64, 64, 0,
                                               LINATTN_FMAP_POLY2, 0, 1, nullptr, nullptr, nullptr, nullptr, P(9), BIG,
                                               nullptr),
                 LINATTN_ERR_SHAPE);
  for (int fm : {-1, 0, 1, 2, 3, INT_MAX})
    for (int nu : {INT_MIN, -1, 0, 1, 3, 4, INT_MAX}) (void)linattn_fmap_dim(fm, nu, 64);

  // ---- delta rule
  CHECK("deltanet ok", deltanet_fwd(P(0), P(1), P(2), P(7), P(3), 4, 8, 4096, 64, 64, 0, F(4), F(4), P(9), BIG,
                                    nullptr),
        LINATTN_OK);
  CHECK("deltanet beta element-aligned", deltanet_fwd(P(0), P(1), P(2), (char*)P(7) + 2, P(3), 4, 8, 4096, 64, 64, 1,
                                                      nullptr, nullptr, P(9), BIG, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("deltanet beta misaligned",
                 deltanet_fwd(P(0), P(1), P(2), (char*)P(7) + 2, P(3), 4, 8, 4096, 64, 64, 0, nullptr, nullptr, P(9),
                              BIG, nullptr),
                 LINATTN_ERR_ALIGN);
  CHECK_NOLAUNCH("deltanet W partial overlap",
                 deltanet_fwd(P(0), P(1), P(2), P(7), P(3), 4, 8, 4096, 64, 64, 0, F(4), F(4) + 4, P(9), BIG,
                              nullptr),
                 LINATTN_ERR_ALIAS);
  CHECK("deltanet step ok", deltanet_decode_step(P(0), P(1), P(2), P(7), P(3), F(4), 256, 16, 64, 64, 1, nullptr),
        LINATTN_OK);
  CHECK_NOLAUNCH("deltanet step W aliases o",
                 deltanet_decode_step(P(0), P(1), P(2), P(7), P(3), (float*)P(3), 256, 16, 64, 64, 1, nullptr),
                 LINATTN_ERR_ALIAS);

  for (int s = -2; s < 12; ++s)
    if (!linattn_status_str(s)) {
      fprintf(stderr, "FAIL status string %d\n", s);
      ++g_fail;
    }
  if (linattn_abi_version() != LINATTN_ABI_VERSION) ++g_fail;
  if (g_fail) {
    fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  printf("abi validation: all cases passed (%d launches)\n", g_launches);
  return 0;
}
