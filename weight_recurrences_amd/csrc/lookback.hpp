// Decoupled look-back for the single-pass causal kernels on gfx950: the block
// states published in the workspace, the per-block flags, and the exclusive
// prefix of a block ("Transformers are RNNs", §3.3 eq.(10)-(11): the prefix
// states are plain sums, so blocks combine by addition).
//
// Every block of a head publishes its increment (the state of its own tokens),
// and some publish their inclusive prefix.  A block's exclusive prefix is the
// left fold S0 + a_0 + ... + a_{b-1} of the increments: it starts from the
// nearest published inclusive prefix and adds the increments after it in order.
// Flags hold (epoch << 8 | producer XCD << 2 | status), fresh per launch, so the
// workspace never needs clearing; a bounded spin falls back to computing a
// missing increment from the inputs, so no wait can hang.
#pragma once

#include <algorithm>
#include <map>
#include <mutex>

#include "common.hpp"
#include "lds_tiles.hpp"

namespace la {
namespace fused {

template <int D, int M>
struct G {
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int WPT = 4 / TD;    // waves sharing a d-tile of S
  static constexpr int TMW = TM / WPT;  // m-tiles of S per wave
  static constexpr int UK = D / 8;      // 16-byte units per K row
  static constexpr int UV = M / 8;      // 16-byte units per V row
  // A published state is the register image of the block's tiles: for every
  // (wave, tile, pair of accumulator rows) 64 lane-consecutive float pairs,
  // followed by z [D].  Producer and consumers own the same tiles.
  static constexpr int SIMG = 4 * TMW * 4 * 64;                        // floats of the S image
  static constexpr int SLOT = ((SIMG + D) * 4 + 255) / 256 * 256;      // bytes per published state
};

// Publish / read a block state in the workspace: S [D][M] then z [D] (float32).
template <int D, int M>
struct Tiles {
  f32x4 S[G<D, M>::TMW];
  f32x4 Z;
};

template <int D, int M>
__device__ __forceinline__ void tiles_zero(Tiles<D, M>& t) {
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) t.S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  t.Z = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D, int M>
__device__ __forceinline__ void tile_coords(int w, int u, int& td, int& tm) {
  td = w % G<D, M>::TD;
  tm = (w / G<D, M>::TD) + G<D, M>::WPT * u;
}

// Published states and flags are written and read with relaxed atomics, so
// publishing needs no cache-wide writeback or invalidate: the producer waits for
// its stores to complete before its flag store, the consumer reads after seeing
// the flag.  Flags are always agent-scope (coherent across the XCDs' L2 caches;
// a poll never hits a stale cached copy).  States:
//  * LOCAL (every block of a head runs on one XCD): workgroup-scope accesses.
//    The stores land in the XCD's L2 and the loads are served from it, so a
//    state never makes a round trip to memory before it is read.  They may hit
//    the reading CU's L1, which is safe: a slot is written once per launch
//    before any reader sees its flag, and the L1 caches are invalidated when a
//    kernel starts.  Each flag carries the producer's XCC id and a consumer
//    accepts only flags from its own XCD, so a placement that breaks the
//    assumption sends the look-back to its fallback, never to stale data.
//  * otherwise agent-scope accesses.
constexpr int FLAG_SCOPE = __HIP_MEMORY_SCOPE_AGENT;
template <bool LOCAL>
struct Scope {
  static constexpr int value = LOCAL ? __HIP_MEMORY_SCOPE_WORKGROUP : __HIP_MEMORY_SCOPE_AGENT;
};

// XCC (XCD) id of the executing wave, from the HW_REG_XCC_ID hardware register.
__device__ __forceinline__ int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 63u); }

// Flag word: epoch (56 bits) << 8 | producer XCC id << 2 | status.
constexpr unsigned long long EPOCH_MASK = (1ull << 56) - 1;
__device__ __forceinline__ unsigned long long flag_word(unsigned long long epoch, int xcc, unsigned long long st) {
  return (epoch << 8) | ((unsigned long long)xcc << 2) | st;
}
// Status of a flag for this launch (0 unless the epoch matches and, for LOCAL
// exchange, the producer ran on the reader's XCD).
template <bool LOCAL>
__device__ __forceinline__ int flag_status(unsigned long long f, unsigned long long epoch, int xcc) {
  const bool ok = (f >> 8) == epoch && (!LOCAL || (int)((f >> 2) & 63ull) == xcc);
  return ok ? (int)(f & 3ull) : 0;
}
__device__ __forceinline__ unsigned long long f2_bits(float a, float b) {
  return (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
}

template <int D, int M, bool LOCAL>
__device__ __forceinline__ void slot_store(char* slot, const Tiles<D, M>& t, int w, int lane, int n, int g) {
  using GG = G<D, M>;
  unsigned long long* s = reinterpret_cast<unsigned long long*>(slot);
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u)
#pragma unroll
    for (int rp = 0; rp < 2; ++rp)
      __hip_atomic_store(&s[((w * GG::TMW + u) * 2 + rp) * 64 + lane], f2_bits(t.S[u][2 * rp], t.S[u][2 * rp + 1]),
                         __ATOMIC_RELAXED, Scope<LOCAL>::value);
  if (w < GG::TD && n == 0) {
    unsigned* z = reinterpret_cast<unsigned*>(slot) + GG::SIMG;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_store(&z[16 * w + 4 * g + r], __float_as_uint(t.Z[r]), __ATOMIC_RELAXED, Scope<LOCAL>::value);
  }
}

template <int D, int M, bool LOCAL>
__device__ __forceinline__ void slot_load(Tiles<D, M>& t, const char* slot, int w, int lane, int g) {
  using GG = G<D, M>;
  unsigned long long* s = reinterpret_cast<unsigned long long*>(const_cast<char*>(slot));
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u)
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      const unsigned long long x =
          __hip_atomic_load(&s[((w * GG::TMW + u) * 2 + rp) * 64 + lane], __ATOMIC_RELAXED, Scope<LOCAL>::value);
      t.S[u][2 * rp] = __uint_as_float((unsigned)x);
      t.S[u][2 * rp + 1] = __uint_as_float((unsigned)(x >> 32));
    }
  t.Z = f32x4{0.f, 0.f, 0.f, 0.f};
  if (w < GG::TD) {
    unsigned* z = reinterpret_cast<unsigned*>(const_cast<char*>(slot)) + GG::SIMG;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      t.Z[r] = __uint_as_float(__hip_atomic_load(&z[16 * w + 4 * g + r], __ATOMIC_RELAXED, Scope<LOCAL>::value));
  }
}

template <int D, int M>
__device__ __forceinline__ void tiles_acc(Tiles<D, M>& a, const Tiles<D, M>& b) {
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) a.S[u] += b.S[u];
  a.Z += b.Z;
}

// Block increments.  EXACT: float32, as slot_store / slot_load.  Otherwise
// S is published as bf16 (8 bytes per lane and tile, half the float32 image) and
// z as float32: the increments then only feed the bf16 S^T operand of the
// outputs.  A block adds its own increment to an inclusive prefix in the same
// rounded form (round_increment), so every fold of the same increments gives
// the same bits.
template <int D, int M, bool EXACT>
__device__ __forceinline__ void round_increment(Tiles<D, M>& t) {
  if (EXACT) return;
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) {
    const uint32_t a = cvt_pk(t.S[u][0], t.S[u][1]), b = cvt_pk(t.S[u][2], t.S[u][3]);
    t.S[u] = f32x4{lo_of(a), hi_of(a), lo_of(b), hi_of(b)};
  }
}

template <int D, int M, bool LOCAL, bool EXACT>
__device__ __forceinline__ void agg_store(char* slot, const Tiles<D, M>& t, int w, int lane, int n, int g) {
  using GG = G<D, M>;
  if (EXACT) {
    slot_store<D, M, LOCAL>(slot, t, w, lane, n, g);
    return;
  }
  unsigned long long* s = reinterpret_cast<unsigned long long*>(slot);
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    const unsigned long long x = (unsigned long long)cvt_pk(t.S[u][0], t.S[u][1]) |
                                 ((unsigned long long)cvt_pk(t.S[u][2], t.S[u][3]) << 32);
    __hip_atomic_store(&s[(w * GG::TMW + u) * 64 + lane], x, __ATOMIC_RELAXED, Scope<LOCAL>::value);
  }
  if (w < GG::TD && n == 0) {
    unsigned* z = reinterpret_cast<unsigned*>(slot) + GG::SIMG;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_store(&z[16 * w + 4 * g + r], __float_as_uint(t.Z[r]), __ATOMIC_RELAXED, Scope<LOCAL>::value);
  }
}

template <int D, int M, bool LOCAL, bool EXACT>
__device__ __forceinline__ void agg_load(Tiles<D, M>& t, const char* slot, int w, int lane, int g) {
  using GG = G<D, M>;
  if (EXACT) {
    slot_load<D, M, LOCAL>(t, slot, w, lane, g);
    return;
  }
  unsigned long long* s = reinterpret_cast<unsigned long long*>(const_cast<char*>(slot));
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    const unsigned long long x = __hip_atomic_load(&s[(w * GG::TMW + u) * 64 + lane], __ATOMIC_RELAXED, Scope<LOCAL>::value);
    const uint32_t a = (uint32_t)x, b = (uint32_t)(x >> 32);
    t.S[u] = f32x4{lo_of(a), hi_of(a), lo_of(b), hi_of(b)};
  }
  t.Z = f32x4{0.f, 0.f, 0.f, 0.f};
  if (w < GG::TD) {
    unsigned* z = reinterpret_cast<unsigned*>(const_cast<char*>(slot)) + GG::SIMG;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      t.Z[r] = __uint_as_float(__hip_atomic_load(&z[16 * w + 4 * g + r], __ATOMIC_RELAXED, Scope<LOCAL>::value));
  }
}

// Adds this wave's elements of a caller state (S [D][M], z [D]).
template <int D, int M>
__device__ __forceinline__ void tiles_add_from_state(Tiles<D, M>& t, const float* S, const float* z, int w, int n,
                                                     int g) {
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) {
    int td, tm;
    tile_coords<D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) t.S[u][r] += S[(16 * td + 4 * g + r) * M + 16 * tm + n];
  }
  if (w < G<D, M>::TD) {
#pragma unroll
    for (int r = 0; r < 4; ++r) t.Z[r] += z[16 * w + 4 * g + r];
  }
}

template <int D, int M>
__device__ __forceinline__ void tiles_store(const Tiles<D, M>& t, float* S, float* z, int w, int n, int g) {
#pragma unroll
  for (int u = 0; u < G<D, M>::TMW; ++u) {
    int td, tm;
    tile_coords<D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[(16 * td + 4 * g + r) * M + 16 * tm + n] = t.S[u][r];
  }
  if (w < G<D, M>::TD && n == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) z[16 * w + 4 * g + r] = t.Z[r];
  }
}

// Exact float32 increment of block p computed straight from global memory
// (the look-back fallback; never needed when predecessors make progress).
template <int D, int M, typename TIn>
__device__ void block_increment_direct(Tiles<D, M>& acc, const TIn* kh, const TIn* vh, int t0, int t1, int w, int n,
                                       int g) {
  for (int j = t0; j < t1; ++j) {
#pragma unroll
    for (int u = 0; u < G<D, M>::TMW; ++u) {
      int td, tm;
      tile_coords<D, M>(w, u, td, tm);
      const float vm = ld_scalar<TIn>(vh + (size_t)j * M + 16 * tm + n);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.S[u][r] += phi(ld_scalar<TIn>(kh + (size_t)j * D + 16 * td + 4 * g + r)) * vm;
    }
    if (w < G<D, M>::TD) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.Z[r] += phi(ld_scalar<TIn>(kh + (size_t)j * D + 16 * w + 4 * g + r));
    }
  }
}

__device__ __forceinline__ unsigned long long rt_clock() { return __builtin_amdgcn_s_memrealtime(); }

// Phase 2 of a single-pass causal kernel: the exclusive prefix P of block b of
// head bh, and the publication of the block's own state.  On entry the block has
// stored its increment L (agg_store, when b > 0 or agg0); this publishes the
// increment's flag, then:
// P_b is the left fold S0 + a_0 + a_1 + ... + a_{b-1} of the block
// increments a_j, evaluated in that order whatever the timing: the block
// starts from the nearest published inclusive prefix (itself such a fold)
// and adds the later increments in forward order.  Results are therefore
// bitwise repeatable; only the never-expected fallback (a predecessor that
// publishes nothing within the spin bound) computes increments differently.
// Every incl_period-th block (and the last) then publishes its inclusive prefix
// P + L (the last block writes it to S_out, z_out when given).  status: an int
// in LDS; kh, vh: the head's keys and values (the fallback's inputs); blocks are
// tblk tokens long; after_publish() runs once the increment's flag is out (or at
// once, for a block that publishes none).  The fold keeps FOLD state loads in
// flight.  Every thread of the workgroup calls
// this.
template <int D, int M, bool LOCAL, bool EXACT, int FOLD, typename TIn, typename AfterPublish>
__device__ __forceinline__ void block_prefix(Tiles<D, M>& P, const Tiles<D, M>& L, int& status, const TIn* kh,
                                             const TIn* vh, int N, int tblk, int b, int bh, int nblk, const float* S0,
                                             const float* z0, float* S_out, float* z_out, unsigned long long* flags,
                                             char* agg_ws, char* incl_ws, unsigned long long epoch,
                                             unsigned long long spin_ticks, int incl_period, bool agg0, int xcc,
                                             int tid, int w, int lane, int n, int g, AfterPublish&& after_publish) {
  using GG = G<D, M>;
  const size_t slot = (size_t)bh * nblk + b;
  tiles_zero<D, M>(P);
  if (agg0 || b > 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&flags[slot], flag_word(epoch, xcc, 1ull), __ATOMIC_RELAXED, FLAG_SCOPE);
  }
  // The caller's loads for after the look-back go out now: they are in flight
  // while the predecessors are awaited.
  after_publish();
  if (b > 0) {
    // Wave 0 polls up to 64 predecessors at once: it needs the nearest one
    // with an inclusive prefix and every block after it with its increment.
    if (w == 0) {
      const int W = b < 64 ? b : 64;
      const unsigned long long inwin = W >= 64 ? ~0ull : ((1ull << W) - 1);
      // -4: timeout; -3: no inclusive prefix within the window; -1: none at all,
      // every predecessor back to block 0 has its increment (fold from S0)
      int pstar = -4;
      const unsigned long long start = rt_clock();
      for (int it = 0; it < (1 << 20); ++it) {
        int st = 0;
        if (lane < W) {
          const unsigned long long f =
              __hip_atomic_load(&flags[(size_t)bh * nblk + (b - 1 - lane)], __ATOMIC_RELAXED, FLAG_SCOPE);
          st = flag_status<LOCAL>(f, epoch, xcc);
        }
        const unsigned long long incl = __ballot(st == 2) & inwin;
        const unsigned long long ready = __ballot(st >= 1) & inwin;
        const int first = incl ? __builtin_ctzll(incl) : W;
        const unsigned long long need = first >= 64 ? inwin : ((1ull << first) - 1);
        if ((ready & need) == need) {
          pstar = first < W ? b - 1 - first : W == b ? -1 : -3;
          break;
        }
        if (rt_clock() - start > spin_ticks) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) status = pstar;
    }
    __syncthreads();
    const int pstar = status;
    if (pstar >= -1) {
      if (pstar >= 0) slot_load<D, M, LOCAL>(P, incl_ws + ((size_t)bh * nblk + pstar) * GG::SLOT, w, lane, g);
      else if (S0) tiles_add_from_state<D, M>(P, S0 + (size_t)bh * D * M, z0 + (size_t)bh * D, w, n, g);
      int j = pstar + 1;
      for (; j + FOLD <= b; j += FOLD) {  // FOLD loads in flight, added in order
        Tiles<D, M> a[FOLD];
#pragma unroll
        for (int f = 0; f < FOLD; ++f)
          agg_load<D, M, LOCAL, EXACT>(a[f], agg_ws + ((size_t)bh * nblk + j + f) * GG::SLOT, w, lane, g);
#pragma unroll
        for (int f = 0; f < FOLD; ++f) tiles_acc<D, M>(P, a[f]);
      }
      for (; j < b; ++j) {
        Tiles<D, M> a0;
        agg_load<D, M, LOCAL, EXACT>(a0, agg_ws + ((size_t)bh * nblk + j) * GG::SLOT, w, lane, g);
        tiles_acc<D, M>(P, a0);
      }
    } else {
      // Slow path: walk back one block at a time with a bounded wait each,
      // computing an increment directly when its block has published nothing.
      bool done = false;
      for (int p = b - 1; p >= 0 && !done; --p) {
        __syncthreads();  // everyone has read status
        if (tid == 0) {
          int st = 0;
          const unsigned long long start = rt_clock();
          for (int it = 0; it < (1 << 20); ++it) {
            const unsigned long long f =
                __hip_atomic_load(&flags[(size_t)bh * nblk + p], __ATOMIC_RELAXED, FLAG_SCOPE);
            if (flag_status<LOCAL>(f, epoch, xcc) != 0) {
              st = flag_status<LOCAL>(f, epoch, xcc);
              break;
            }
            if (rt_clock() - start > spin_ticks) break;
            __builtin_amdgcn_s_sleep(2);
          }
          status = st;
        }
        __syncthreads();
        const int st = status;
        const size_t ps = (size_t)bh * nblk + p;
        Tiles<D, M> a0;
        if (st == 2) {
          slot_load<D, M, LOCAL>(a0, incl_ws + ps * GG::SLOT, w, lane, g);
          done = true;
        } else if (st == 1) {
          agg_load<D, M, LOCAL, EXACT>(a0, agg_ws + ps * GG::SLOT, w, lane, g);
        } else {
          tiles_zero<D, M>(a0);
          block_increment_direct<D, M>(a0, kh, vh, p * tblk, min(N, (p + 1) * tblk), w, n, g);
          round_increment<D, M, EXACT>(a0);
        }
        tiles_acc<D, M>(P, a0);
      }
      if (!done && S0) tiles_add_from_state<D, M>(P, S0 + (size_t)bh * D * M, z0 + (size_t)bh * D, w, n, g);
    }
  } else if (S0) {
    tiles_add_from_state<D, M>(P, S0 + (size_t)bh * D * M, z0 + (size_t)bh * D, w, n, g);
  }

  // Inclusive prefixes are published by every incl_period-th block only (the
  // last one of each group of that many consecutive blocks of a head, which is
  // all of a head that is resident at once); the blocks after it fold the
  // increments from there.  Every published prefix is the same left fold, so
  // the results do not depend on which one a block finds.
  if (b == nblk - 1 || b % incl_period == incl_period - 1) {
    Tiles<D, M> inc = L;
    round_increment<D, M, EXACT>(inc);  // the increment as the successors fold it
#pragma unroll
    for (int u = 0; u < GG::TMW; ++u) inc.S[u] = P.S[u] + inc.S[u];
    inc.Z = P.Z + inc.Z;
    if (b == nblk - 1) {
      if (S_out) tiles_store<D, M>(inc, S_out + (size_t)bh * D * M, z_out + (size_t)bh * D, w, n, g);
    } else {
      slot_store<D, M, LOCAL>(incl_ws + slot * GG::SLOT, inc, w, lane, n, g);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(&flags[slot], flag_word(epoch, xcc, 2ull), __ATOMIC_RELAXED, FLAG_SCOPE);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
struct WsLayout {
  size_t flags_bytes, slot_bytes, init_bytes, total;
};

template <int D, int M>
static WsLayout layout(long long BH, int N, int tblk) {
  const long long nblk = (N + tblk - 1) / tblk;
  WsLayout l;
  l.flags_bytes = (size_t)((BH * nblk * 8 + 255) / 256 * 256);
  l.slot_bytes = (size_t)G<D, M>::SLOT;
  // private copy of an initial state that the call overwrites in place
  l.init_bytes = (size_t)((BH * (D * M + D) * 4 + 255) / 256 * 256);
  l.total = l.flags_bytes + 2 * (size_t)(BH * nblk) * l.slot_bytes + l.init_bytes;
  return l;
}

// Launch epochs: strictly increasing across calls and, being seeded from the
// wall clock, across processes, so flags left in a reused workspace by any
// earlier launch never match the current one (one counter for every kernel
// that uses the look-back).
unsigned long long lookback_epoch();

// Workgroups of a kernel resident at once on the current device (cached).
static inline int resident_wgs(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 512;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per <= 0) per = 1;
  return cache[key] = cus * per;
}

}  // namespace fused
}  // namespace la
