// Host check of the LDS address split used by the bf16 causal kernel: for every
// access site of that kernel (every lane, wave, chunk, slab and tile it uses, at
// every built (D, M)), the address formed from a per-lane part and compile-time
// parts equals the swizzled address 2 * swz<U>(row, col) of the element.
// Prints "ok" and exits 0, or prints the first mismatch and exits 1.
#include <cstdio>

#include "lds_tiles.hpp"

using la::lane_off;
using la::swz;
using la::xor_off;

static int fails = 0;
static void expect(unsigned got, int want, const char* site, int a, int b, int c, int d) {
  if (got != (unsigned)want && fails++ == 0)
    std::printf("mismatch at %s (%d %d %d %d): %u != %d\n", site, a, b, c, d, got, want);
}

template <int D, int M>
static void check() {
  constexpr int NT = 256, CH = 64, NCH = 4;
  constexpr int UK = D / 8, UV = M / 8, TD = D / 16, TM = M / 16, WPT = 4 / TD, TMW = TM / WPT;
  constexpr int KV = CH * D * 2 / 16 / NT, VV = CH * M * 2 / 16 / NT, QV = D / 32;
  for (int tid = 0; tid < NT; ++tid) {
    const int w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16, td = w % TD;
    const unsigned l_kst = lane_off<UK>(tid / UK, 8 * (tid % UK));
    const unsigned l_vst = lane_off<UV>(tid / UV, 8 * (tid % UV));
    const unsigned l_trv = lane_off<UV>(4 * g + (n >> 2), 4 * (n & 3));
    const unsigned l_trk_w = lane_off<UK>(4 * g + (n >> 2), 4 * (n & 3)) ^ xor_off<UK>(16 * td);
    const unsigned l_trv_w = l_trv ^ xor_off<UV>(16 * (w / TD));
    const unsigned l_rd = lane_off<UK>(n, 8 * g);
    const unsigned l_wr = lane_off<UK>(n, 4 * g);
    for (int c = 0; c < NCH; ++c) {
      // unit stores of the loaded K (resident tile and staging tile) and V rows
      for (int i = 0; i < KV; ++i) {
        const int p = tid + NT * i, R = c * CH + i * (NT / UK);
        expect(16 * UK * R + (l_kst ^ xor_off<UK>(0)), 2 * swz<UK>(c * CH + p / UK, (p % UK) * 8), "K store", D, M, tid, c);
        const int R0 = i * (NT / UK);
        expect(16 * UK * R0 + (l_kst ^ xor_off<UK>(0)), 2 * swz<UK>(p / UK, (p % UK) * 8), "K tail store", D, M, tid, c);
      }
      for (int i = 0; i < VV; ++i) {
        const int p = tid + NT * i, R = c * CH + i * (NT / UV);
        expect(16 * UV * R + (l_vst ^ xor_off<UV>(0)), 2 * swz<UV>(c * CH + p / UV, (p % UV) * 8), "V store", D, M, tid, c);
      }
      for (int s = 0; s < CH / 32; ++s)
        for (int h = 0; h < 2; ++h) {
          const int R = c * CH + 32 * s + 16 * h, row = R + 4 * g + (n >> 2);
          // transposed reads: phi(K) d-tile td, and the tail staging tile
          expect(16 * UK * R + (l_trk_w ^ xor_off<UK>(0)), 2 * swz<UK>(row, 16 * td + 4 * (n & 3)), "K tr", D, M, tid, c);
          const int Rs = 32 * s + 16 * h;
          expect(16 * UK * Rs + (l_trk_w ^ xor_off<UK>(0)), 2 * swz<UK>(Rs + 4 * g + (n >> 2), 16 * td + 4 * (n & 3)), "K tail tr", D, M, tid, c);
          // V m-tiles of phase 1 (this wave's) and of phase 3 (all)
          for (int u = 0; u < TMW; ++u) {
            const int tm = w / TD + WPT * u, C = 16 * WPT * u;
            expect(16 * UV * R + (l_trv_w ^ xor_off<UV>(C)), 2 * swz<UV>(row, 16 * tm + 4 * (n & 3)), "V tr 1", D, M, tid, c);
          }
          for (int tm = 0; tm < TM; ++tm)
            expect(16 * UV * R + (l_trv ^ xor_off<UV>(16 * tm)), 2 * swz<UV>(row, 16 * tm + 4 * (n & 3)), "V tr 3", D, M, tid, c);
        }
      // score operand reads
      for (int t = 0; t < 4; ++t)
        for (int s = 0; s < QV; ++s) {
          const int R = c * CH + 16 * t;
          expect(16 * UK * R + (l_rd ^ xor_off<UK>(32 * s)), 2 * swz<UK>(R + n, 32 * s + 8 * g), "score", D, M, tid, c);
        }
    }
    // state operand reads and writes
    for (int tm = 0; tm < TM; ++tm)
      for (int s = 0; s < QV; ++s)
        expect(16 * UK * 16 * tm + (l_rd ^ xor_off<UK>(32 * s)), 2 * swz<UK>(16 * tm + n, 32 * s + 8 * g), "St read", D, M, tid, tm);
    for (int u = 0; u < TMW; ++u) {
      const int tdd = w % TD, tm = w / TD + WPT * u;
      expect(16 * UK * 16 * tm + (l_wr ^ xor_off<UK>(16 * tdd)), 2 * swz<UK>(16 * tm + n, 16 * tdd + 4 * g), "St write", D, M, tid, u);
    }
  }
}

int main() {
  check<32, 32>();
  check<32, 64>();
  check<64, 32>();
  check<64, 64>();
  if (fails) {
    std::printf("%d mismatches\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
