// Causal and non-causal linear attention on gfx950 (MI355X).
//
// Method: "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器": phi = elu + 1 (§3.2.1 eq.(7)); causal form by prefix states
// S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j),
// o_i = phi(q_i)^T S_i / phi(q_i)^T z_i (§3.3 eq.(9)-(12)); non-causal form by
// associativity (§3.2 eq.(5)-(6)).
//
// Chunked evaluation.  The sequence of each (batch, head) is cut into chunks of
// CH = 64 tokens.  For a chunk c with the state (S, z) of everything before it:
//   num_i = phi(q_i)^T S + sum_{j in c, j<=i} (phi(q_i).phi(k_j)) v_j
//   den_i = phi(q_i)^T z + sum_{j in c, j<=i}  phi(q_i).phi(k_j)
//   o_i = num_i / den_i, then S += phi(K_c)^T V_c, z += column sums of phi(K_c).
// This is eq.(9) with the prefix sum split at the chunk boundary; every
// product is a dense 16x16 MFMA tile contraction.  To fill the GPU, each head's
// sequence is further cut into blocks of several chunks: one kernel computes
// each block's state increment, a scan kernel turns them into exclusive
// prefixes (eq.(10)-(11) are plain sums, so blocks combine by addition), and
// the sweep kernel runs the chunk recurrence of each block from its prefix.
//
// Workgroup: 4 wavefronts.  Wave w owns query rows [16w, 16w+16) of a chunk and
// a fixed set of 16x16 tiles of S.  Lane l = 16*g + n (n = l % 16, g = l / 16).
//
// Operand layouts (MFMA 16x16x32 bf16 / 16x16x4 f32):
//  * contraction over d (feature dim): lane group g holds d-slots
//      bf16: d = 32*s + 8*g + e (e < 8) for slab s;  f32: d = (D/4)*g + s.
//  * contraction over j (tokens of a chunk): lane group g holds
//      bf16: j = 32*s + 16*h + 4*g + r (e = 4h + r) — exactly the rows that the
//      lane holds in an accumulator tile, so a masked score tile becomes an A
//      operand without data movement;  f32: j = 16*t + 4*g + r for slab (t, r).
//  * value columns are interleaved: B-operand column n of m-tile tm is
//    m = TM*n + tm, so a lane ends up with TM consecutive output columns.
//
// Precision.  bf16 MFMA operands carry 8 significant bits.  Scores, P and the
// inter-chunk S operand only feed the bf16 output, so one bf16 rounding is
// enough there.  The state update S += phi(K)^T V feeds the float32 state, so
// phi(K) is split into a bf16 head and tail (phi = hi + lo to ~2^-17) and both
// are multiplied by the exact bf16 V: the state then carries float32-level
// error.  z uses the same split, and its operand for the denominator is split
// the same way.
//
// LDS per workgroup of the sweep kernel (bf16, D=M=64: 45.3 KiB, three
// workgroups per CU; f32: 52.5 KiB):
//   Kr  [CH][D]  phi(K) row-major (bf16 path; A operand of the score tiles)
//   Kt  [D][CH]  phi(K) transposed (A operand of the state update)
//   Ktl [D][CH]  tail of phi(K) - Kt (bf16 path only)
//   Vt  [M][CH]  V transposed (B operand of P.V and of the state update)
//   St  [M][D]   S^T in the operand precision
//   Zs  [D]      z in float32
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {

constexpr int CH = 64;   // chunk length
constexpr int NT = 256;  // threads per workgroup

template <typename T, int D, int M>
struct CG {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int WPT = 4 / TD;     // waves sharing one d-tile of S
  static constexpr int TMW = TM / WPT;   // m-tiles of S owned by one wave
  static constexpr int PAD = BF ? 8 : 4;
  static constexpr int SKR = D + PAD;
  static constexpr int SKT = CH + PAD;
  static constexpr int SST = D + PAD;
  static constexpr int NSD = BF ? D / 32 : D / 4;  // d-slabs
  static constexpr int EPV = 16 / sizeof(T);       // elements per 16-byte vector
};

// Sweep kernel: everything.
template <typename T, int D, int M>
struct Smem {
  using G = CG<T, D, M>;
  static constexpr bool HAS_KR = G::BF;
  T Kr[G::BF ? CH * G::SKR : 4];
  T Kt[D * G::SKT];
  T Ktl[G::BF ? D * G::SKT : 4];
  T Vt[M * G::SKT];
  T St[M * G::SST];
  float Zs[D];
};

// Block-state kernel: only the operands of the state update.
template <typename T, int D, int M>
struct SmemState {
  using G = CG<T, D, M>;
  static constexpr bool HAS_KR = false;
  T Kr[4];
  T Kt[D * G::SKT];
  T Ktl[G::BF ? D * G::SKT : 4];
  T Vt[M * G::SKT];
};

// Non-causal apply kernel: only the state.
template <typename T, int D, int M>
struct SmemApply {
  using G = CG<T, D, M>;
  T St[M * G::SST];
  float Zs[D];
};

// ----------------------------------------------------------------------------
// Global -> register tile of CH rows x W elements (16-byte vectors, coalesced).
template <typename T, int W>
struct Tile {
  static constexpr int VPR = W * (int)sizeof(T) / 16;  // vectors per row
  static constexpr int NV = CH * VPR / NT;              // vectors per thread
  u32x4 v[NV];
};

template <typename T, int W>
__device__ __forceinline__ void tile_load(Tile<T, W>& t, const T* rows, int nvalid, int tid) {
#pragma unroll
  for (int u = 0; u < Tile<T, W>::NV; ++u) {
    const int p = tid + NT * u;
    const int row = p / Tile<T, W>::VPR, c = p % Tile<T, W>::VPR;
    if (row < nvalid)
      t.v[u] = *reinterpret_cast<const u32x4*>(rows + (size_t)row * W + c * (16 / sizeof(T)));
    else
      t.v[u] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ float vec_elem_f(const u32x4& v, int e, float) { return __uint_as_float(v[e]); }
__device__ __forceinline__ float vec_elem_b(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return bf2f((e & 1) ? (w >> 16) : (w & 0xffffu));
}

template <typename T> __device__ __forceinline__ float vec_elem(const u32x4& v, int e);
template <> __device__ __forceinline__ float vec_elem<float>(const u32x4& v, int e) { return __uint_as_float(v[e]); }
template <> __device__ __forceinline__ float vec_elem<bf16_t>(const u32x4& v, int e) { return vec_elem_b(v, e); }

// phi(K) tile -> Kr (bf16 path) and Kt; rows >= nvalid become exact zeros so
// that padding contributes nothing to S, z or the scores.
template <typename T, int D, int M, typename SM>
__device__ __forceinline__ void store_k(SM& sm, const Tile<T, D>& t, int nvalid, int tid) {
  using G = CG<T, D, M>;
#pragma unroll
  for (int u = 0; u < Tile<T, D>::NV; ++u) {
    const int p = tid + NT * u;
    const int row = p / Tile<T, D>::VPR, c = p % Tile<T, D>::VPR;
    const bool ok = row < nvalid;
    float f[G::EPV];
#pragma unroll
    for (int e = 0; e < G::EPV; ++e) f[e] = ok ? phi(vec_elem<T>(t.v[u], e)) : 0.f;
    if constexpr (G::BF) {
      uint32_t hb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hb[e] = f2bf(f[e]);
      if constexpr (SM::HAS_KR) {
        u32x4 pk{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
        *reinterpret_cast<u32x4*>(&sm.Kr[row * G::SKR + c * 8]) = pk;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sm.Kt[(c * 8 + e) * G::SKT + row] = (bf16_t)hb[e];
        sm.Ktl[(c * 8 + e) * G::SKT + row] = (bf16_t)f2bf(f[e] - bf2f(hb[e]));
      }
    } else {
#pragma unroll
      for (int e = 0; e < G::EPV; ++e) sm.Kt[(c * G::EPV + e) * G::SKT + row] = f[e];
    }
  }
}

template <typename T, int D, int M, typename SM>
__device__ __forceinline__ void store_v(SM& sm, const Tile<T, M>& t, int tid) {
  using G = CG<T, D, M>;
#pragma unroll
  for (int u = 0; u < Tile<T, M>::NV; ++u) {
    const int p = tid + NT * u;
    const int row = p / Tile<T, M>::VPR, c = p % Tile<T, M>::VPR;
    if constexpr (G::BF) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = t.v[u][e >> 1];
        sm.Vt[(c * 8 + e) * G::SKT + row] = (bf16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Vt[(c * 4 + e) * G::SKT + row] = __uint_as_float(t.v[u][e]);
    }
  }
}

// ----------------------------------------------------------------------------
// Fragments.
template <typename T, int D>
struct QFrag {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NSD = BF ? D / 32 : D / 4;
  typename std::conditional<BF, bf16x8, float>::type f[NSD];
};

// Raw query bits of one row, prefetched a chunk ahead; phi is applied only
// when the chunk is processed (so the prefetch never stalls on its loads).
template <typename T, int D>
struct QRaw {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NV = BF ? D / 32 : D / 16;  // 16-byte vectors per lane
  u32x4 v[NV];
  bool ok;
};

// Loads the d-slots of query row `row` (zeros when row >= nvalid):
// bf16 vector s holds d = 32s + 8g .. +7; f32 vector c holds d = (D/4)g + 4c .. +3.
template <typename T, int D>
__device__ __forceinline__ void load_q(QRaw<T, D>& qr, const T* q, int row, int nvalid, int g) {
  qr.ok = row < nvalid;
#pragma unroll
  for (int s = 0; s < QRaw<T, D>::NV; ++s) {
    const int off = QRaw<T, D>::BF ? 32 * s + 8 * g : (D / 4) * g + 4 * s;
    qr.v[s] = qr.ok ? *reinterpret_cast<const u32x4*>(q + (size_t)row * D + off) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T, int D>
__device__ __forceinline__ void q_phi(QFrag<T, D>& qf, const QRaw<T, D>& qr) {
  if constexpr (QFrag<T, D>::BF) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 pk;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t w = qr.v[s][h];
        const float a = qr.ok ? phi(bf2f(w & 0xffffu)) : 0.f;
        const float b = qr.ok ? phi(bf2f(w >> 16)) : 0.f;
        pk[h] = pack_bf2(a, b);
      }
      qf.f[s] = as_bf16x8(pk);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) qf.f[4 * c + e] = qr.ok ? phi(__uint_as_float(qr.v[c][e])) : 0.f;
  }
}

__device__ __forceinline__ bf16x8 ones_bf16x8() {
  const uint32_t one2 = 0x3F803F80u;
  return as_bf16x8(u32x4{one2, one2, one2, one2});
}

// bf16 j-slot fragment of a transposed tile row (Kt or Vt): slots
// j = 32s + 16h + 4g + r, taken as two 8-byte reads.
template <int SKT>
__device__ __forceinline__ bf16x8 jfrag_bf16(const bf16_t* trow, int s, int g) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(trow + 32 * s + 4 * g);
  const u32x2 b = *reinterpret_cast<const u32x2*>(trow + 32 * s + 16 + 4 * g);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// ----------------------------------------------------------------------------
// State held by one wave: its tiles of S (fp32 accumulators) and, for waves
// w < TD, the matching d-tile of z.
template <typename T, int D, int M>
struct WaveState {
  using G = CG<T, D, M>;
  f32x4 S[G::TMW];
  f32x4 Z;
};

template <typename T, int D, int M>
__device__ __forceinline__ void state_coords(int w, int u, int& td, int& tm) {
  using G = CG<T, D, M>;
  td = w % G::TD;
  tm = (w / G::TD) + G::WPT * u;
}

// Load this wave's tiles of (S, z) from a [D][M] / [D] fp32 state (or zero).
template <typename T, int D, int M>
__device__ __forceinline__ void state_load(WaveState<T, D, M>& st, const float* S, const float* z, int w, int n, int g) {
  using G = CG<T, D, M>;
#pragma unroll
  for (int u = 0; u < G::TMW; ++u) {
    int td, tm;
    state_coords<T, D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) st.S[u][r] = S ? S[(16 * td + 4 * g + r) * M + G::TM * n + tm] : 0.f;
  }
  const int td = w % G::TD;
#pragma unroll
  for (int r = 0; r < 4; ++r) st.Z[r] = (z && w < G::TD) ? z[16 * td + 4 * g + r] : 0.f;
}

template <typename T, int D, int M>
__device__ __forceinline__ void state_store(const WaveState<T, D, M>& st, float* S, float* z, int w, int n, int g) {
  using G = CG<T, D, M>;
#pragma unroll
  for (int u = 0; u < G::TMW; ++u) {
    int td, tm;
    state_coords<T, D, M>(w, u, td, tm);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[(16 * td + 4 * g + r) * M + G::TM * n + tm] = st.S[u][r];
  }
  if (w < G::TD && n == 0) {
    const int td = w;
#pragma unroll
    for (int r = 0; r < 4; ++r) z[16 * td + 4 * g + r] = st.Z[r];
  }
}

// Publish this wave's tiles of S (operand precision, transposed) and z.
template <typename T, int D, int M, typename SM>
__device__ __forceinline__ void state_to_lds(const WaveState<T, D, M>& st, SM& sm, int w, int n, int g) {
  using G = CG<T, D, M>;
#pragma unroll
  for (int u = 0; u < G::TMW; ++u) {
    int td, tm;
    state_coords<T, D, M>(w, u, td, tm);
    T* dst = &sm.St[(G::TM * n + tm) * G::SST + 16 * td + 4 * g];
    if constexpr (G::BF) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(st.S[u][0], st.S[u][1]), pack_bf2(st.S[u][2], st.S[u][3])};
    } else {
      *reinterpret_cast<f32x4*>(dst) = st.S[u];
    }
  }
  if (w < G::TD && n == 0) *reinterpret_cast<f32x4*>(&sm.Zs[16 * w + 4 * g]) = st.Z;
}

// S += phi(K_c)^T V_c and z += column sums of phi(K_c), for this wave's tiles.
template <typename T, int D, int M, typename SM>
__device__ __forceinline__ void state_update(WaveState<T, D, M>& st, const SM& sm, int w, int n, int g) {
  using G = CG<T, D, M>;
  const int td = w % G::TD;
  const T* krow = &sm.Kt[(16 * td + n) * G::SKT];
  if constexpr (G::BF) {
    const bf16x8 ones = ones_bf16x8();
    const T* krowl = &sm.Ktl[(16 * td + n) * G::SKT];
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      const bf16x8 a = jfrag_bf16<G::SKT>(krow, s, g);
      const bf16x8 al = jfrag_bf16<G::SKT>(krowl, s, g);
#pragma unroll
      for (int u = 0; u < G::TMW; ++u) {
        int tdd, tm;
        state_coords<T, D, M>(w, u, tdd, tm);
        const bf16x8 b = jfrag_bf16<G::SKT>(&sm.Vt[(G::TM * n + tm) * G::SKT], s, g);
        st.S[u] = mma(a, b, st.S[u]);
        st.S[u] = mma(al, b, st.S[u]);
      }
      if (w < G::TD) {
        st.Z = mma(a, ones, st.Z);
        st.Z = mma(al, ones, st.Z);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < CH / 16; ++t) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + 16 * t + 4 * g);
      f32x4 b4[G::TMW];
#pragma unroll
      for (int u = 0; u < G::TMW; ++u) {
        int tdd, tm;
        state_coords<T, D, M>(w, u, tdd, tm);
        b4[u] = *reinterpret_cast<const f32x4*>(&sm.Vt[(G::TM * n + tm) * G::SKT + 16 * t + 4 * g]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int u = 0; u < G::TMW; ++u) st.S[u] = mma(a4[r], b4[u][r], st.S[u]);
        if (w < G::TD) st.Z = mma(a4[r], 1.f, st.Z);
      }
    }
  }
}

// Eight float32 z values -> bf16 head and tail operands (z = hi + lo to ~2^-17).
__device__ __forceinline__ void z_split(const float* z8, bf16x8& zh, bf16x8& zl) {
  const f32x4 z0 = *reinterpret_cast<const f32x4*>(z8);
  const f32x4 z1 = *reinterpret_cast<const f32x4*>(z8 + 4);
  const float zz[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
  uint32_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = f2bf(zz[e]);
    lb[e] = f2bf(zz[e] - bf2f(hb[e]));
  }
  zh = as_bf16x8(u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)});
  zl = as_bf16x8(u32x4{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16), lb[6] | (lb[7] << 16)});
}

// o_i = num_i / den_i for the 16 rows of wave w: lane (n, g) holds rows
// 16w + 4g + r and the TM consecutive columns TM*n .. TM*n + TM - 1.
template <typename T, int M>
__device__ __forceinline__ void store_rows(T* o, const f32x4* num, const f32x4& den, int nvalid, int w, int n, int g) {
  constexpr int TM = M / 16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * g + r;
    if (i < nvalid) {
      const float inv = 1.f / den[r];
      T* dst = o + (size_t)i * M + TM * n;
      if constexpr (sizeof(T) == 2) {
        if constexpr (TM == 4) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(num[0][r] * inv, num[1][r] * inv), pack_bf2(num[2][r] * inv, num[3][r] * inv)};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = pack_bf2(num[0][r] * inv, num[1][r] * inv);
        }
      } else {
        if constexpr (TM == 4) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{num[0][r] * inv, num[1][r] * inv, num[2][r] * inv, num[3][r] * inv};
        } else {
          *reinterpret_cast<float2*>(dst) = float2{num[0][r] * inv, num[1][r] * inv};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Outputs of one chunk for this wave's 16 query rows.
template <typename T, int D, int M>
__device__ __forceinline__ void chunk_outputs(const Smem<T, D, M>& sm, const QFrag<T, D>& qf,
                                              T* o, int nvalid, int w, int n, int g) {
  using G = CG<T, D, M>;
  f32x4 num[G::TM];
#pragma unroll
  for (int tm = 0; tm < G::TM; ++tm) num[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 den{0.f, 0.f, 0.f, 0.f};

  // Scores A^T[j][i] = phi(k_j).phi(q_i) for j-tiles t <= w (tiles above the
  // diagonal are entirely masked by j <= i).
  f32x4 at[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    at[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t <= w) {
      if constexpr (G::BF) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.Kr[(16 * t + n) * G::SKR + 32 * s + 8 * g]));
          at[t] = mma(a, qf.f[s], at[t]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < D / 4; ++s) {
          const float a = sm.Kt[((D / 4) * g + s) * G::SKT + 16 * t + n];
          at[t] = mma(a, qf.f[s], at[t]);
        }
      }
      if (t == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r > n) at[t][r] = 0.f;  // inclusive causal mask j <= i
      }
    }
  }

  // Intra-chunk part: num += P V, den += P 1.
  if constexpr (G::BF) {
    const bf16x8 ones = ones_bf16x8();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (2 * s <= w) {
        const bf16x8 p = as_bf16x8(u32x4{pack_bf2(at[2 * s][0], at[2 * s][1]), pack_bf2(at[2 * s][2], at[2 * s][3]),
                                         pack_bf2(at[2 * s + 1][0], at[2 * s + 1][1]),
                                         pack_bf2(at[2 * s + 1][2], at[2 * s + 1][3])});
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm) {
          const bf16x8 b = jfrag_bf16<G::SKT>(&sm.Vt[(G::TM * n + tm) * G::SKT], s, g);
          num[tm] = mma(p, b, num[tm]);
        }
        den = mma(p, ones, den);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t <= w) {
        f32x4 b4[G::TM];
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm)
          b4[tm] = *reinterpret_cast<const f32x4*>(&sm.Vt[(G::TM * n + tm) * G::SKT + 16 * t + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int tm = 0; tm < G::TM; ++tm) num[tm] = mma(at[t][r], b4[tm][r], num[tm]);
          den = mma(at[t][r], 1.f, den);
        }
      }
    }
  }

  // Inter-chunk part: num += phi(Q) S, den += phi(Q) z.
  if constexpr (G::BF) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.St[(G::TM * n + tm) * G::SST + 32 * s + 8 * g]));
        num[tm] = mma(qf.f[s], b, num[tm]);
      }
      bf16x8 zh, zl;
      z_split(&sm.Zs[32 * s + 8 * g], zh, zl);
      den = mma(qf.f[s], zh, den);
      den = mma(qf.f[s], zl, den);
    }
  } else {
#pragma unroll
    for (int s = 0; s < D / 4; ++s) {
      const int d = (D / 4) * g + s;
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm) num[tm] = mma(qf.f[s], sm.St[(G::TM * n + tm) * G::SST + d], num[tm]);
      den = mma(qf.f[s], sm.Zs[d], den);
    }
  }

  store_rows<T, M>(o, num, den, nvalid, w, n, g);
}

// ----------------------------------------------------------------------------
// Kernel 1: state increment of every block (grid: BH * nblk, blockIdx.x = bh * nblk + blk).
//   agg[bh][blk] = sum_{j in block} phi(k_j) v_j^T,  aggz[bh][blk] = sum phi(k_j).
// With add_base != 0 (single-block mode) the base state (S_base, z_base; NULL
// for zero) is added and the result written to agg/aggz at slot bh.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void block_state_kernel(const T* __restrict__ k, const T* __restrict__ v, int N,
                                                         int tblk, int nblk, float* agg, float* aggz,
                                                         const float* S_base, const float* z_base, int add_base) {
  __shared__ SmemState<T, D, M> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int blk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const T* kh = k + ((size_t)bh * N) * D;
  const T* vh = v + ((size_t)bh * N) * M;

  WaveState<T, D, M> st;
  if (add_base)
    state_load<T, D, M>(st, S_base ? S_base + (size_t)bh * D * M : nullptr, z_base ? z_base + (size_t)bh * D : nullptr, w, n, g);
  else
    state_load<T, D, M>(st, nullptr, nullptr, w, n, g);

  Tile<T, D> tk;
  Tile<T, M> tv;
  tile_load<T, D>(tk, kh + (size_t)t0 * D, t1 - t0, tid);
  tile_load<T, M>(tv, vh + (size_t)t0 * M, t1 - t0, tid);
  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    store_k<T, D, M>(sm, tk, nv, tid);
    store_v<T, D, M>(sm, tv, tid);
    __syncthreads();
    if (c0 + CH < t1) {
      const int nn = min(CH, t1 - c0 - CH);
      tile_load<T, D>(tk, kh + (size_t)(c0 + CH) * D, nn, tid);
      tile_load<T, M>(tv, vh + (size_t)(c0 + CH) * M, nn, tid);
    }
    state_update<T, D, M>(st, sm, w, n, g);
    __syncthreads();
  }
  const size_t slot = add_base ? (size_t)bh : (size_t)bh * nblk + blk;
  state_store<T, D, M>(st, agg + slot * D * M, aggz + slot * D, w, n, g);
}

// Kernel 3: chunk sweep with outputs (grid: BH * nblk, blockIdx.x = bh * nblk + blk).
// The block starts from the state in (Sp, zp): per block when per_block != 0,
// else per head (NULL for zero).  With S_fin != NULL the block's final state is
// written there (per head).
//
// Per chunk: [publish S^T, z; store phi(K), V tiles] barrier [phi(Q); issue the
// next chunk's loads; outputs; state update] barrier.  Between the barriers
// every wave only reads LDS, so the next chunk's tiles and the new S^T are
// written after the second barrier.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void causal_sweep_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, T* __restrict__ o, int N, int tblk,
                                                          int nblk, const float* Sp, const float* zp, int per_block,
                                                          float* S_fin, float* z_fin) {
  __shared__ Smem<T, D, M> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int blk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const T* qh = q + ((size_t)bh * N) * D;
  const T* kh = k + ((size_t)bh * N) * D;
  const T* vh = v + ((size_t)bh * N) * M;
  T* oh = o + ((size_t)bh * N) * M;

  Tile<T, D> tk;
  Tile<T, M> tv;
  QRaw<T, D> qr;
  tile_load<T, D>(tk, kh + (size_t)t0 * D, t1 - t0, tid);
  tile_load<T, M>(tv, vh + (size_t)t0 * M, t1 - t0, tid);
  load_q<T, D>(qr, qh + (size_t)t0 * D, 16 * w + n, t1 - t0, g);

  const size_t slot = per_block ? (size_t)bh * nblk + blk : (size_t)bh;
  WaveState<T, D, M> st;
  state_load<T, D, M>(st, Sp ? Sp + slot * D * M : nullptr, zp ? zp + slot * D : nullptr, w, n, g);

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    state_to_lds<T, D, M>(st, sm, w, n, g);
    store_k<T, D, M>(sm, tk, nv, tid);
    store_v<T, D, M>(sm, tv, tid);
    __syncthreads();
    QFrag<T, D> qf;
    q_phi<T, D>(qf, qr);
    if (c0 + CH < t1) {
      const int nn = min(CH, t1 - c0 - CH);
      tile_load<T, D>(tk, kh + (size_t)(c0 + CH) * D, nn, tid);
      tile_load<T, M>(tv, vh + (size_t)(c0 + CH) * M, nn, tid);
      load_q<T, D>(qr, qh + (size_t)(c0 + CH) * D, 16 * w + n, nn, g);
    }
    chunk_outputs<T, D, M>(sm, qf, oh + (size_t)c0 * M, nv, w, n, g);
    state_update<T, D, M>(st, sm, w, n, g);
    __syncthreads();
  }
  if (S_fin) state_store<T, D, M>(st, S_fin + (size_t)bh * D * M, z_fin + (size_t)bh * D, w, n, g);
}

// Kernel 2: per-head scan over blocks (grid: BH * ceil((DM+D)/NT)).
// exclusive != 0: agg[b] <- S_init + sum_{b' < b} agg[b'] in place (causal).
// The total S_init + sum_b agg[b] goes to (S_tot, z_tot) when non-NULL.
__global__ __launch_bounds__(NT) void state_scan_kernel(float* agg, float* aggz, int nblk, int DM, int D,
                                                        const float* S_init, const float* z_init, float* S_tot,
                                                        float* z_tot, int exclusive) {
  const int parts = (DM + D + NT - 1) / NT;
  const int e = (blockIdx.x % parts) * NT + threadIdx.x, bh = blockIdx.x / parts;
  if (e >= DM + D) return;
  const bool isz = e >= DM;
  const int x = isz ? e - DM : e;
  const int len = isz ? D : DM;
  float* base = (isz ? aggz : agg) + (size_t)bh * nblk * len + x;
  const float* init = isz ? z_init : S_init;
  float run = init ? init[(size_t)bh * len + x] : 0.f;
  // Eight records per round are loaded before any is written, so the loads are
  // in flight together; the sums still run in block order.
  constexpr int U = 8;
  int b = 0;
  for (; b + U <= nblk; b += U) {
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = base[(size_t)(b + u) * len];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (exclusive) base[(size_t)(b + u) * len] = run;
      run += t[u];
    }
  }
  for (; b < nblk; ++b) {
    const float t = base[(size_t)b * len];
    if (exclusive) base[(size_t)b * len] = run;
    run += t;
  }
  float* tot = isz ? z_tot : S_tot;
  if (tot) tot[(size_t)bh * len + x] = run;
}

// Copies (S_init, z_init) to (S_out, z_out), or zero-fills them (empty sequence).
__global__ __launch_bounds__(NT) void state_copy_kernel(const float* S_init, const float* z_init, float* S_out,
                                                        float* z_out, long long nS, long long nz) {
  const long long e = (long long)blockIdx.x * NT + threadIdx.x;
  if (e < nS) S_out[e] = S_init ? S_init[e] : 0.f;
  if (e < nz) z_out[e] = z_init ? z_init[e] : 0.f;
}

// Non-causal apply (grid: BH * nblk, blockIdx.x = bh * nblk + blk):
// o_i = phi(q_i)^T S / phi(q_i)^T z with the head's full-sequence state.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void noncausal_apply_kernel(const T* __restrict__ q, T* __restrict__ o, int N,
                                                             int tblk, int nblk, const float* S, const float* z) {
  __shared__ SmemApply<T, D, M> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int blk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  using G = CG<T, D, M>;
  const T* qh = q + ((size_t)bh * N) * D;
  T* oh = o + ((size_t)bh * N) * M;
  QRaw<T, D> qr;
  load_q<T, D>(qr, qh + (size_t)t0 * D, 16 * w + n, t1 - t0, g);
  {
    WaveState<T, D, M> st;
    state_load<T, D, M>(st, S + (size_t)bh * D * M, z + (size_t)bh * D, w, n, g);
    state_to_lds<T, D, M>(st, sm, w, n, g);
  }
  __syncthreads();
  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    QFrag<T, D> qf;
    q_phi<T, D>(qf, qr);
    if (c0 + CH < t1) load_q<T, D>(qr, qh + (size_t)(c0 + CH) * D, 16 * w + n, min(CH, t1 - c0 - CH), g);
    f32x4 num[G::TM];
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm) num[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 den{0.f, 0.f, 0.f, 0.f};
    if constexpr (G::BF) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm) {
          const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.St[(G::TM * n + tm) * G::SST + 32 * s + 8 * g]));
          num[tm] = mma(qf.f[s], b, num[tm]);
        }
        bf16x8 zh, zl;
        z_split(&sm.Zs[32 * s + 8 * g], zh, zl);
        den = mma(qf.f[s], zh, den);
        den = mma(qf.f[s], zl, den);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 4; ++s) {
        const int d = (D / 4) * g + s;
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm) num[tm] = mma(qf.f[s], sm.St[(G::TM * n + tm) * G::SST + d], num[tm]);
        den = mma(qf.f[s], sm.Zs[d], den);
      }
    }
    store_rows<T, M>(oh + (size_t)c0 * M, num, den, nv, w, n, g);
  }
}

// ----------------------------------------------------------------------------
// Host-side launchers.
int causal_block_tokens(int BH, int N) {
  if (N <= 0 || BH <= 0) return CH;
  const int per_head = BH >= 1024 ? 1 : (1024 + BH - 1) / BH;
  int tb = (N + per_head - 1) / per_head;
  tb = ((tb + CH - 1) / CH) * CH;
  if (tb < 256) tb = 256;
  const int ncap = ((N + CH - 1) / CH) * CH;
  if (tb > ncap) tb = ncap;
  return tb;
}

template <typename T, int D, int M>
static hipError_t causal_impl(const void* q, const void* k, const void* v, void* o, int BH, int N,
                              const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                              hipStream_t stream) {
  const int tblk = causal_block_tokens(BH, N);
  const int nblk = (N + tblk - 1) / tblk;
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(NT);
  const T* qq = (const T*)q;
  const T* kk = (const T*)k;
  const T* vv = (const T*)v;
  if (nblk == 1) {
    if (o) {
      hipLaunchKernelGGL((causal_sweep_kernel<T, D, M>), grid, block, 0, stream, qq, kk, vv, (T*)o, N, tblk, 1, S0,
                         z0, 0, S_out, z_out);
    } else {
      hipLaunchKernelGGL((block_state_kernel<T, D, M>), grid, block, 0, stream, kk, vv, N, tblk, 1, S_out, z_out,
                         S0, z0, 1);
    }
    return hipGetLastError();
  }
  float* agg = (float*)ws;
  float* aggz = agg + (size_t)BH * nblk * D * M;
  hipLaunchKernelGGL((block_state_kernel<T, D, M>), grid, block, 0, stream, kk, vv, N, tblk, nblk, agg, aggz,
                     nullptr, nullptr, 0);
  const dim3 sgrid((unsigned)((D * M + D + NT - 1) / NT) * (unsigned)BH);
  hipLaunchKernelGGL(state_scan_kernel, sgrid, block, 0, stream, agg, aggz, nblk, D * M, D, S0, z0, S_out, z_out,
                     1);
  if (o)
    hipLaunchKernelGGL((causal_sweep_kernel<T, D, M>), grid, block, 0, stream, qq, kk, vv, (T*)o, N, tblk, nblk, agg,
                       aggz, 1, nullptr, nullptr);
  return hipGetLastError();
}

template <typename T, int D, int M>
static hipError_t noncausal_impl(const void* q, const void* k, const void* v, void* o, int BH, int N, void* ws,
                                 hipStream_t stream) {
  const int tblk = causal_block_tokens(BH, N);
  const int nblk = (N + tblk - 1) / tblk;
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(NT);
  float* agg = (float*)ws;
  float* aggz = agg + (size_t)BH * nblk * D * M;
  float* Stot = aggz + (size_t)BH * nblk * D;
  float* ztot = Stot + (size_t)BH * D * M;
  hipLaunchKernelGGL((block_state_kernel<T, D, M>), grid, block, 0, stream, (const T*)k, (const T*)v, N, tblk, nblk,
                     agg, aggz, nullptr, nullptr, 0);
  const dim3 sgrid((unsigned)((D * M + D + NT - 1) / NT) * (unsigned)BH);
  hipLaunchKernelGGL(state_scan_kernel, sgrid, block, 0, stream, agg, aggz, nblk, D * M, D, nullptr, nullptr, Stot,
                     ztot, 0);
  hipLaunchKernelGGL((noncausal_apply_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, (T*)o, N, tblk, nblk,
                     Stot, ztot);
  return hipGetLastError();
}

// Exclusive prefix state of every block of T = tblk tokens (agg [BH][nblk][D][M],
// aggz [BH][nblk][D]), from a zero initial state; used by the backward pass.
template <typename T, int D, int M>
static hipError_t block_prefix_impl(const void* k, const void* v, int BH, int N, int tblk, int nblk, float* agg,
                                    float* aggz, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {  // bf16: the bf16-MFMA block kernel of the non-causal path
    const hipError_t e = launch_block_state_bf16(k, v, BH, N, D, M, tblk, nblk, agg, aggz, stream);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((block_state_kernel<T, D, M>), dim3((unsigned)nblk * (unsigned)BH), dim3(NT), 0, stream,
                       (const T*)k, (const T*)v, N, tblk, nblk, agg, aggz, nullptr, nullptr, 0);
  }
  const dim3 sgrid((unsigned)((D * M + D + NT - 1) / NT) * (unsigned)BH);
  hipLaunchKernelGGL(state_scan_kernel, sgrid, dim3(NT), 0, stream, agg, aggz, nblk, D * M, D, nullptr, nullptr,
                     nullptr, nullptr, 1);
  return hipGetLastError();
}

hipError_t launch_block_prefix(const void* k, const void* v, int BH, int N, int D, int M, int bf16, int tblk,
                               int nblk, float* agg, float* aggz, hipStream_t stream) {
  if (bf16) {
    LA_DISPATCH_DM(block_prefix_impl, bf16_t, k, v, BH, N, tblk, nblk, agg, aggz, stream)
  } else {
    LA_DISPATCH_DM(block_prefix_impl, float, k, v, BH, N, tblk, nblk, agg, aggz, stream)
  }
}

hipError_t launch_state_scan(float* agg, float* aggz, int BHs, int nblk, int DM, int D, const float* S_init,
                             const float* z_init, float* S_tot, float* z_tot, int exclusive, hipStream_t stream) {
  const dim3 sgrid((unsigned)((DM + D + NT - 1) / NT) * (unsigned)BHs);
  hipLaunchKernelGGL(state_scan_kernel, sgrid, dim3(NT), 0, stream, agg, aggz, nblk, DM, D, S_init, z_init, S_tot,
                     z_tot, exclusive);
  return hipGetLastError();
}

hipError_t launch_state_copy(const float* S_init, const float* z_init, float* S_out, float* z_out, long long nS,
                             long long nz, hipStream_t stream) {
  const unsigned nb = (unsigned)(((nS > nz ? nS : nz) + NT - 1) / NT);
  hipLaunchKernelGGL(state_copy_kernel, dim3(nb), dim3(NT), 0, stream, S_init, z_init, S_out, z_out, nS, nz);
  return hipGetLastError();
}

// Causal calls take the single-pass kernels (causal_fused.hip for bf16,
// causal_fused32.hip for float32) unless LINATTN_CAUSAL_PATH=blocked selects the
// three-kernel path (kept for comparisons).  Read at every call, by the
// workspace query and by the launch alike.
static bool causal_fused_path() {
  const char* e = getenv("LINATTN_CAUSAL_PATH");
  return !(e && strcmp(e, "blocked") == 0);
}

size_t causal_ws_bytes(int BH, int N, int D, int M, int bf16) {
  if (BH <= 0 || N <= 0) return 0;
  if (causal_fused_path()) return bf16 ? causal_fused_ws_bytes(BH, N, D, M) : causal_fused32_ws_bytes(BH, N, D, M);
  const int tblk = causal_block_tokens(BH, N);
  const long long nblk = (N + tblk - 1) / tblk;
  if (nblk <= 1) return 0;
  return (size_t)BH * nblk * (size_t)(D * M + D) * sizeof(float);
}

size_t noncausal_ws_bytes(int BH, int N, int D, int M, int bf16) {
  if (BH <= 0 || N <= 0) return 0;
  if (bf16) return noncausal_bf16_ws_bytes(BH, N, D, M);
  const int tblk = causal_block_tokens(BH, N);
  const long long nblk = (N + tblk - 1) / tblk;
  return (size_t)BH * (nblk + 1) * (size_t)(D * M + D) * sizeof(float);
}

hipError_t launch_causal(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                         int bf16, const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                         hipStream_t stream) {
  if (N == 0) {
    if (!S_out) return hipSuccess;
    const long long nS = (long long)BH * D * M, nz = (long long)BH * D;
    const unsigned nb = (unsigned)((nS + NT - 1) / NT);
    hipLaunchKernelGGL(state_copy_kernel, dim3(nb), dim3(NT), 0, stream, S0, z0, S_out, z_out, nS, nz);
    return hipGetLastError();
  }
  if (causal_fused_path()) {
    if (bf16) return launch_causal_fused(q, k, v, o, BH, N, D, M, S0, z0, S_out, z_out, ws, stream);
    return launch_causal_fused32(q, k, v, o, BH, N, D, M, S0, z0, S_out, z_out, ws, stream);
  }
  if (bf16) {
    LA_DISPATCH_DM(causal_impl, bf16_t, q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream)
  } else {
    LA_DISPATCH_DM(causal_impl, float, q, k, v, o, BH, N, S0, z0, S_out, z_out, ws, stream)
  }
}

hipError_t launch_noncausal(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                            int bf16, void* ws, hipStream_t stream) {
  if (bf16) return launch_noncausal_bf16(q, k, v, o, BH, N, D, M, ws, stream);
  LA_DISPATCH_DM(noncausal_impl, float, q, k, v, o, BH, N, ws, stream)
}

}  // namespace la
