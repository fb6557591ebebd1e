// Chunk-parallel delta rule on gfx950.
//
// News summary of "Linear Transformers Are Secretly Fast Weight Programmers"
// (Schlag, Irie, Schmidhuber, 2021), paragraphs on the new update rule and on
// normalisation: per token, kh = phi(k)/sum phi(k), qh likewise,
// vbar = W kh, W += beta (v - vbar) kh^T, o = W qh (the updated memory).
//
// The same recurrence, regrouped by chunks of C = 64 tokens (exact up to
// rounding).  With W0 the memory at the chunk start, the values actually written,
// u_t = beta_t (v_t - W_{t-1} kh_t), satisfy
//   u_t + beta_t sum_{s<t} (kh_t . kh_s) u_s = beta_t (v_t - W0 kh_t),
// a unit lower-triangular system.  With G = Kh Kh^T, L its strictly lower part
// and B = diag(beta): U = T (V - Kh W0^T), T = (I + B L)^{-1} B, and
//   o_t = W0 qh_t + sum_{s<=t} (qh_t . kh_s) u_s,   W_end = W0 + U^T Kh.
// T depends on the keys and beta only, so every chunk's T is formed in parallel.
//
// The update of row m of W involves only row m (and the shared kh, beta), so a
// head's memory splits into slices of 16 rows that evolve independently.
//
// Two kernels:
//   dn_prep_kernel   per (head, chunk), all in parallel: kh, G (split-bf16 MFMA)
//                    and T in fp32 (16x16x4 MFMA): the four diagonal 16x16 blocks of T by
//                    substitution, the blocks below them by doubling,
//                    T_ab = -T_aa G_ab T_bb for 16-row blocks, then the same for
//                    the 32-row halves.  Writes kh and T as bf16 head and tail
//                    (below), laid out as the chain kernel uses them.
//   dn_chain_kernel  per (head, 16-row slice of W): the chunks in order, the
//                    slice in registers.  Per chunk: R = V - Kh W^T, U = T R,
//                    W^T += Kh^T U; for token tile w of the chunk,
//                    o_w = Qh_w W_{<w}^T + tril(Qh_w Kh_w^T) U_w with W_{<w} the
//                    memory after the chunk's tiles before w (the score terms with
//                    earlier tiles folded into it: sum_{j<w} (Qh_w Kh_j^T) U_j =
//                    Qh_w (sum_{j<w} U_j^T Kh_j)).
// The chain's products are bf16 MFMA (16x16x32) on operands split into a bf16
// head and tail (x = h + l to about 2^-17 relative), as h h + h l + l h with fp32
// accumulation (the tail x tail term, about 2^-16 of a product, is dropped); the
// memory itself stays fp32 in the accumulators across the chunks.  A wave64
// VALU instruction takes four cycles, so the sequential kernel keeps its VALU
// work small: kh arrives already split and in its LDS layout (a plain copy), T
// already split in MFMA operand order; only qh is formed there.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace la {
namespace dnc {

constexpr int NT = 256;    // threads per workgroup (4 wavefronts)
constexpr int C = 64;      // tokens per chunk

// ---- bf16 head/tail operands ------------------------------------------------
// Four floats -> {head01, head23, tail01, tail23} (round to nearest even).
__device__ __forceinline__ u32x4 split4(f32x4 x) {
  const uint32_t h0 = cvt_pk(x[0], x[1]), h1 = cvt_pk(x[2], x[3]);
  return u32x4{h0, h1, cvt_pk(x[0] - lo_of(h0), x[1] - hi_of(h0)), cvt_pk(x[2] - lo_of(h1), x[3] - hi_of(h1))};
}
// Eight floats -> eight-element head and tail operands.
__device__ __forceinline__ void split8(const float (&x)[8], u32x4& h, u32x4& l) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = cvt_pk(x[2 * i], x[2 * i + 1]);
    l[i] = cvt_pk(x[2 * i] - lo_of(h[i]), x[2 * i + 1] - hi_of(h[i]));
  }
}
// Raw buffer resource over [p, p + bytes): stores at offsets past the end are
// discarded by the hardware (the third-word flags are the 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, bytes, 0x00020000);
}
template <typename T> __device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int off, float x);
template <> __device__ __forceinline__ void store_elem<float>(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
template <> __device__ __forceinline__ void store_elem<bf16_t>(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2bf(x), r, off, 0, 0);
}

// c + a b with a = ah + al, b = bh + bl: three bf16 products.
__device__ __forceinline__ f32x4 mma3(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
  c = mma(as_bf16x8(ah), as_bf16x8(bh), c);
  c = mma(as_bf16x8(ah), as_bf16x8(bl), c);
  return mma(as_bf16x8(al), as_bf16x8(bh), c);
}

// ----------------------------------------------------------------------------
// Per-chunk record in the workspace (16-byte units), for chunk (bh, c) at unit
// (bh * nch + c) * Rec<D>::UNITS:
//   [0, KI)         kh as the chain kernel's two bf16 LDS tiles (head, then
//                   tail): row-major [t][d], 16-byte units swizzled (lds_tiles.hpp);
//   [KI, KI + 768)  T in operand order: for block b = (w, sg) of the six
//                   (token tile w, slab sg <= w / 2) pairs, lane l = 16 g + n
//                   holds T[16 w + n][32 sg + 16 h + 4 g + r] (e = 4 h + r) as a
//                   head unit then a tail unit at 128 b + 2 l.
template <int D>
struct Rec {
  static constexpr int U8 = D / 8;          // 16-byte units per bf16 row
  static constexpr int KI = 2 * C * U8;     // kh image units (head and tail)
  static constexpr int UNITS = KI + 6 * 128;
};
__host__ __device__ constexpr int t_block(int w, int sg) { return w < 2 ? w : 2 * w - 2 + sg; }

// ----------------------------------------------------------------------------
// Grid BH * nch, blockIdx.x = bh * nch + c.
// MFMA 16x16x4 f32 (lane l = 16 g + n): a = A[n][k], b = B[k][n] for the k-slot
// g; the accumulator holds D[4 g + r][n] in element r.
// G and T live in LDS as their ten 16x16 blocks on and below the diagonal only,
// row stride 17 inside a block (lb below).
__device__ __forceinline__ int lb(int r, int c) {  // (r, c) with c / 16 <= r / 16
  const int i = r >> 4, j = c >> 4;
  return (i * (i + 1) / 2 + j) * 272 + (r & 15) * 17 + (c & 15);
}

template <typename T, int D>
__global__ __launch_bounds__(NT, 4) void dn_prep_kernel(const T* __restrict__ k, const T* __restrict__ beta, int N,
                                                        int nch, u32x4* __restrict__ ws) {
  using RR = Rec<D>;
  constexpr int UPR = D / 4;
  constexpr int U8 = RR::U8;
  constexpr int SL = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ki[2][C * D];  // kh head and tail, swizzled (the chain's layout)
  __shared__ float Gs[10 * 272];
  __shared__ float Ts[10 * 272];
  __shared__ float Bs[C];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int t0 = c * C, nt = min(C, N - t0);
  u32x4* rec = ws + ((size_t)bh * nch + c) * RR::UNITS;

  // kh = phi(k) / sum phi(k), split into head and tail, into LDS and the record;
  // rows at or past nt are zero (their beta is zero too).
  {
    float4 raw[C * UPR / NT];
    const T* src = k + ((size_t)bh * N + t0) * D;
#pragma unroll
    for (int i = 0; i < C * UPR / NT; ++i) {
      const int u = tid + NT * i, row = u / UPR;
      raw[i] = load4<T>(src + (size_t)min(row, nt - 1) * D + (u % UPR) * 4);
    }
    const float bt = ld_scalar<T>(beta + (size_t)bh * N + t0 + min(tid & (C - 1), nt - 1));
    if (tid < C) Bs[tid] = tid < nt ? bt : 0.f;
    u32x2* rec2 = reinterpret_cast<u32x2*>(rec);
#pragma unroll
    for (int i = 0; i < C * UPR / NT; ++i) {
      const int u = tid + NT * i, row = u / UPR, c4 = (u % UPR) * 4;
      f32x4 x{phi(raw[i].x), phi(raw[i].y), phi(raw[i].z), phi(raw[i].w)};
      float s = (x[0] + x[1]) + (x[2] + x[3]);
      s = UPR == 16 ? sum16(s) : sum8(s);
      const float inv = row < nt ? __builtin_amdgcn_rcpf(s) : 0.f;  // 1 ulp
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= inv;
      const u32x4 hl = split4(x);
      const int e8 = swz<U8>(row, c4) >> 2;  // 8-byte half unit
      unit8<U8>(Ki[0], row, c4) = u32x2{hl[0], hl[1]};
      unit8<U8>(Ki[1], row, c4) = u32x2{hl[2], hl[3]};
      rec2[e8] = u32x2{hl[0], hl[1]};
      rec2[2 * C * U8 + e8] = u32x2{hl[2], hl[3]};
    }
  }
  __syncthreads();

  // G blocks on and below the diagonal (d-contraction on split-bf16 MFMA):
  // tile p = i (i + 1) / 2 + j for block (i, j), j <= i; wave w takes p = w, w + 4, w + 8.
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const int p = w + 4 * it;
    const int i = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
    const int j = min(p, 9) - i * (i + 1) / 2;
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SL; ++s)
      acc = mma3(unit16<U8>(Ki[0], 16 * i + n, 32 * s + 8 * g), unit16<U8>(Ki[1], 16 * i + n, 32 * s + 8 * g),
                 unit16<U8>(Ki[0], 16 * j + n, 32 * s + 8 * g), unit16<U8>(Ki[1], 16 * j + n, 32 * s + 8 * g), acc);
    if (p < 10) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Gs[lb(16 * i + 4 * g + r, 16 * j + n)] = acc[r];
    }
  }
  __syncthreads();

  // Diagonal blocks T_ii = (I + B_i L_ii)^{-1} B_i: wave 0, lane (n, g) solves
  // column n of block i = g, x_t = beta_t (e_n - sum_{s<t} G_ts x_s)_t, right-looking.
  if (w == 0) {
    const int base = 16 * g;
    float z[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) z[t] = t == n ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float x = Bs[base + t] * z[t];
      z[t] = x;
#pragma unroll
      for (int t2 = t + 1; t2 < 16; ++t2) z[t2] -= Gs[lb(base + t2, base + t)] * x;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) Ts[lb(base + t, base + n)] = z[t];
  }
  __syncthreads();

  // Below the diagonal, for a lower-triangular [[T_bb, 0], [X, T_aa]] block pair:
  // X = -T_aa G_ab T_bb.  First the 16-row pairs (1, 0) and (3, 2) (waves 0, 1;
  // waves 2, 3 repeat them and discard the result).  The product T_aa Y takes Y
  // from the accumulator with the k-permutation k = 4 g + r.
  {
    const int a = 2 * (w & 1) + 1, b = a - 1;
    f32x4 y{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      y = mma(Gs[lb(16 * a + n, 16 * b + 4 * kk + g)], Ts[lb(16 * b + 4 * kk + g, 16 * b + n)], y);
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) x = mma(Ts[lb(16 * a + n, 16 * a + 4 * g + r)], y[r], x);
    if (w < 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[lb(16 * a + 4 * g + r, 16 * b + n)] = -x[r];
    }
  }
  __syncthreads();
  // Then the 32-row halves: with T_A = T[0:32][0:32], T_B = T[32:64][32:64],
  // T[32:64][0:32] = -T_B (G[32:64][0:32] T_A).  Wave w forms block (2 + a2, c2),
  // a2 = w / 2, c2 = w % 2: -sum_{b2 <= a2} T[2 + a2][2 + b2] Y[b2],
  // Y[b2] = sum_{e >= c2} G[2 + b2][e] T[e][c2] (terms outside the triangles are
  // masked to zero, so every wave runs the same products; a masked term reads a
  // block inside the triangle instead of one outside it).
  {
    const int a2 = w >> 1, c2 = w & 1;
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      f32x4 y{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bool on = e >= c2;
          const float ga = on ? Gs[lb(16 * (2 + b2) + n, 16 * e + 4 * kk + g)] : 0.f;
          const float tb = on ? Ts[lb(16 * e + 4 * kk + g, 16 * (on ? c2 : 0) + n)] : 0.f;
          y = mma(ga, tb, y);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool on = b2 <= a2;
        const float ta = on ? Ts[lb(16 * (2 + a2) + n, 16 * (2 + (on ? b2 : 0)) + 4 * g + r)] : 0.f;
        x = mma(ta, y[r], x);
      }
    }
    // The blocks written here (rows 32.., columns ..31) are read by no wave above.
#pragma unroll
    for (int r = 0; r < 4; ++r) Ts[lb(16 * (2 + a2) + 4 * g + r, 16 * c2 + n)] = -x[r];
  }
  __syncthreads();

  // T in operand order (tiles above the diagonal blocks as zeros).
  for (int i = tid; i < 6 * 64; i += NT) {
    const int b = i >> 6, l = i & 63, ln = l & 15, lg = l >> 4;
    const int bw = b < 2 ? b : 2 + ((b - 2) >> 1), sg = b < 2 ? 0 : (b - 2) & 1;
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = 2 * sg + h <= bw;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[4 * h + r] = ok ? Ts[lb(16 * bw + ln, ok ? 32 * sg + 16 * h + 4 * lg + r : 0)] : 0.f;
    }
    u32x4 h, lo;
    split8(x, h, lo);
    rec[RR::KI + 128 * b + 2 * l] = h;
    rec[RR::KI + 128 * b + 2 * l + 1] = lo;
  }
}

// ----------------------------------------------------------------------------
// The chain.  One workgroup per (head, 16-row slice of W); the NS = M / 16
// slices of a head get workgroup indices equal mod 8, so they share an XCD (and
// its L2) for the q and record reads they have in common.  Grid 8 ceil(BH / 8) NS.
//
// MFMA 16x16x32 bf16 layouts (lane l = 16 g + n; lds_tiles.hpp): a d-contraction
// operand holds d = 32 s + 8 g + e of slab s; a token contraction holds tokens
// 32 s + 16 h + 4 g + r (e = 4 h + r), the rows an accumulator tile keeps in the
// lane, so accumulators feed it directly.
//
// Eight waves, two per SIMD.  Waves 0-3 run the sequential path only: wave w owns
// token tile w (rows 16 w ..) for X, R and U, and the 16-wide d tile w of the
// memory slice (W^T rows 16 w .., fp32 in its accumulator).  Waves 4-7 do the
// work that does not depend on the memory's next value, alongside: the loads,
// staging of the next chunk, the score tiles, P and o for token tile w - 4.
// Per chunk (three barriers):
//   path:   X = Kh W^T (W^T from the slice tile in LDS), R = V - X -> LDS
//   others: loads for later chunks, the last chunk's o stored; P = Qh W^T;
//           score tiles S^T = Kh Qh^T of token tiles 0, 1 (masked to s <= t)
//   | path:   U = T R (token contraction over R of all token tiles) -> LDS
//     others: score tiles 2, 3; kh copied and half of qh staged for the next chunk
//   | path:   W^T += Kh^T U (Kh^T by transposed LDS reads) -> slice tile in LDS
//     others: o = P + S U; the other half of qh staged
//   |
// The products on the sequential path keep their three partial products in
// separate accumulators, so that they do not wait on each other.
__device__ __forceinline__ void mma3s(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 (&c)[3]) {
  c[0] = mma(as_bf16x8(ah), as_bf16x8(bh), c[0]);
  c[1] = mma(as_bf16x8(ah), as_bf16x8(bl), c[1]);
  c[2] = mma(as_bf16x8(al), as_bf16x8(bh), c[2]);
}
__device__ __forceinline__ f32x4 sum3(const f32x4 (&c)[3]) {
  f32x4 x;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = c[0][r] + (c[1][r] + c[2][r]);
  return x;
}

constexpr int NTC = 2 * NT;  // threads of the chain kernel

template <typename T, int D, int M>
__global__ __launch_bounds__(NTC) void dn_chain_kernel(const T* __restrict__ q, const T* __restrict__ v,
                                                       const u32x4* __restrict__ ws, int BH, int N, int nch,
                                                       const float* __restrict__ W0, float* __restrict__ W_out,
                                                       T* __restrict__ o) {
  using RR = Rec<D>;
  constexpr int U8 = RR::U8;  // 16-byte units per bf16 row of D (swizzle width)
  constexpr int TD = D / 16;  // d tiles of the slice
  constexpr int SL = D / 32;  // slabs of a d-contraction
  constexpr int NS = M / 16;  // slices per head
  constexpr int UPR = D / 4;  // 4-element units per row of q
  constexpr int NU = C * UPR / NT;  // q units per helper thread
  constexpr int KU = RR::KI / NT;   // kh image units per helper thread
  __shared__ __attribute__((aligned(16))) bf16_t Kt[2][2][C * D];  // [buffer][head, tail] kh [t][d], swizzled
  __shared__ __attribute__((aligned(16))) bf16_t Qt[2][2][C * D];  // qh
  // The slice [m][d] (head, tail) at the start of chunks of either parity, and
  // after token tiles 0, 1, 2 of the current chunk.
  __shared__ __attribute__((aligned(16))) bf16_t Wt[2][2][16 * D];
  __shared__ __attribute__((aligned(16))) bf16_t Wp[3][2][16 * D];
  __shared__ u32x4 Rx[4][64];                                      // R tiles, per token tile and lane
  __shared__ u32x4 Ux[4][64];                                      // U tiles
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const bool path = __builtin_amdgcn_readfirstlane(wv) < 4;  // the wave's role (a scalar branch)
  const int w = wv & 3, ht = tid & (NT - 1);
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int bh = (jx / NS) * 8 + xcd, m0 = 16 * (jx % NS);
  if (bh >= BH) return;
  const int dt = w % TD;  // d tile of a path wave (waves past TD repeat and discard)

  const T* qb = q + (size_t)bh * N * D;
  const T* vb = v + (size_t)bh * N * M + m0 + n;
  const u32x4* recb = ws + (size_t)bh * nch * RR::UNITS;

  // Raw q of a chunk, units [i0, i1) (rows clamped into the chunk; masked when
  // staged), and its kh image (helper waves).
  auto load_q = [&](int c, float4 (&rq)[NU], int i0, int i1) __attribute__((always_inline)) {
    const int t0 = c * C, last = min(C, N - t0) - 1;
    const T* qc = qb + (size_t)t0 * D;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      if (i < i0 || i >= i1) continue;
      const int u = ht + NT * i;
      rq[i] = load4<T>(qc + min(u / UPR, last) * D + (u % UPR) * 4);
    }
  };
  auto load_k = [&](int c, u32x4 (&rk)[KU]) __attribute__((always_inline)) {
    const u32x4* rc = recb + (size_t)c * RR::UNITS;
#pragma unroll
    for (int i = 0; i < KU; ++i) rk[i] = rc[ht + NT * i];
  };
  auto copy_k = [&](int buf, const u32x4 (&rk)[KU]) __attribute__((always_inline)) {
    u32x4* kd = reinterpret_cast<u32x4*>(Kt[buf][0]);
#pragma unroll
    for (int i = 0; i < KU; ++i) kd[ht + NT * i] = rk[i];
  };
  // phi(q) / sum phi(q) per row, split into head and tail tiles: units [i0, i1).
  auto stage_q = [&](int buf, int c, const float4 (&rq)[NU], int i0, int i1) __attribute__((always_inline)) {
    const int nt = min(C, N - c * C);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      if (i < i0 || i >= i1) continue;
      const int u = ht + NT * i, row = u / UPR, c4 = (u % UPR) * 4;
      const float4 r = rq[i];
      f32x4 x{phi(r.x), phi(r.y), phi(r.z), phi(r.w)};
      float s = (x[0] + x[1]) + (x[2] + x[3]);
      s = UPR == 16 ? sum16(s) : sum8(s);
      const float inv = row < nt ? __builtin_amdgcn_rcpf(s) : 0.f;  // 1 ulp, as for kh
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= inv;
      const u32x4 hl = split4(x);
      unit8<U8>(Qt[buf][0], row, c4) = u32x2{hl[0], hl[1]};
      unit8<U8>(Qt[buf][1], row, c4) = u32x2{hl[2], hl[3]};
    }
  };
  // T of token tile w in operand order (slab 1 of tiles 0 and 1 is zero) and V
  // in the accumulator layout, rows 16 w + 4 g + r, column m0 + n (path waves).
  auto load_tv = [&](int c, u32x4 (&tt)[4], float (&rv)[4]) __attribute__((always_inline)) {
    const u32x4* rc = recb + (size_t)c * RR::UNITS + RR::KI + 2 * lane;
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const u32x4* p = rc + 128 * t_block(w, w < 2 ? 0 : sg);
      tt[2 * sg] = p[0];
      tt[2 * sg + 1] = p[1];
    }
    const int t0 = c * C, last = min(C, N - t0) - 1;
    const T* vc = vb + (size_t)t0 * M;
#pragma unroll
    for (int r = 0; r < 4; ++r) rv[r] = ld_scalar<T>(vc + min(16 * w + 4 * g + r, last) * M);
  };

  // Path wave: the slice's d tile dt, transposed: wm[r] = W[m0 + n][16 dt + 4 g + r].
  // (Every wave loads it and waits for it here: a load left pending on only
  // some paths into the loop would make the compiler wait for all loads in
  // flight at its first use inside the loop, on every chunk.)
  f32x4 wm{0.f, 0.f, 0.f, 0.f};
  if (W0) {
    const float4 x = *reinterpret_cast<const float4*>(W0 + ((size_t)bh * M + m0 + n) * D + 16 * dt + 4 * g);
    wm = f32x4{x.x, x.y, x.z, x.w};
  }
  __builtin_amdgcn_s_waitcnt(0);
  auto put_w = [&](bf16_t (&dst)[2][16 * D], f32x4 x) __attribute__((always_inline)) {
    if (w < TD) {
      const u32x4 hl = split4(x);
      unit8<U8>(dst[0], n, 16 * dt + 4 * g) = u32x2{hl[0], hl[1]};
      unit8<U8>(dst[1], n, 16 * dt + 4 * g) = u32x2{hl[2], hl[3]};
    }
  };

  // Helper wave: outputs of chunk c, formed at the start of chunk c + 1 (after
  // that chunk's loads are issued: loads and stores share one counter, and a
  // store issued before a load makes every later wait for the load wait for it
  // too).  Rows past the chunk fall outside the buffer resource and are
  // dropped, with no branch that would cost the compiler its count of the loads
  // in flight.
  //   o_t = W_{<t} qh_t + sum_{s <= t} (qh_t . kh_s) u_s for t in token tile w
  //       = Qh_w Wa^T + tril(Qh_w Kh_w^T) U_w,
  // with Wa the memory after token tiles 0 .. w - 1 of the chunk (its start for
  // w = 0): the score products with earlier token tiles are folded into Wa,
  // which the path waves form alongside the memory update.
  auto outputs = [&](int c) __attribute__((always_inline)) {  // c < 0: nothing stored (empty resource)
    const int pb = c & 1, t0 = max(c, 0) * C;
    const bf16_t *Kh = Kt[pb][0], *Kl = Kt[pb][1], *Qh = Qt[pb][0], *Ql = Qt[pb][1];
    const bf16_t(&Wa)[2][16 * D] = w == 0 ? Wt[pb] : Wp[w - 1];
    const f32x4 z4{0.f, 0.f, 0.f, 0.f};
    f32x4 O3[3] = {z4, z4, z4}, sacc = z4;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const u32x4 qh = unit16<U8>(Qh, 16 * w + n, 32 * s + 8 * g), ql = unit16<U8>(Ql, 16 * w + n, 32 * s + 8 * g);
      mma3s(qh, ql, unit16<U8>(Wa[0], n, 32 * s + 8 * g), unit16<U8>(Wa[1], n, 32 * s + 8 * g), O3);
      sacc = mma3(unit16<U8>(Kh, 16 * w + n, 32 * s + 8 * g), unit16<U8>(Kl, 16 * w + n, 32 * s + 8 * g), qh, ql,
                  sacc);
    }
    // the diagonal score tile S^T[s][t], s, t in token tile w, masked to s <= t,
    // in half w % 2 of slab w / 2 of a token contraction (the other half zero)
    f32x4 sm;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm[r] = 4 * g + r <= n ? sacc[r] : 0.f;
    const u32x4 shl = split4(sm);
    const bool hi = w & 1;
    const u32x4 sh = hi ? u32x4{0u, 0u, shl[0], shl[1]} : u32x4{shl[0], shl[1], 0u, 0u};
    const u32x4 sl = hi ? u32x4{0u, 0u, shl[2], shl[3]} : u32x4{shl[2], shl[3], 0u, 0u};
    const int sg = w >> 1;
    const u32x4 ua = Ux[2 * sg][lane], ub = Ux[2 * sg + 1][lane];
    mma3s(sh, sl, u32x4{ua[0], ua[1], ub[0], ub[1]}, u32x4{ua[2], ua[3], ub[2], ub[3]}, O3);
    const f32x4 oc = sum3(O3);
    const int bytes = c < 0 ? 0 : min(C, N - t0) * M * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t ob = out_rsrc(o + ((size_t)bh * N + t0) * M, bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) store_elem<T>(ob, ((16 * w + 4 * g + r) * M + m0 + n) * (int)sizeof(T), oc[r]);
  };

  // The two roles run separate loops with the same three barriers per chunk,
  // so that the compiler's count of each wave's loads in flight covers only its
  // own loads (a loop that interleaves both roles' code would make every wait
  // count the other role's loads and stores as well).
  //
  // Path waves.  Chunk c: X and R; U; the memory update.  On entry (tt, rv) hold
  // chunk c's T and V; chunk c + 1's are loaded into (tt2, rv2).
  auto path_chunk = [&](int c, const u32x4 (&tt)[4], const float (&rv)[4], u32x4 (&tt2)[4], float (&rv2)[4])
                        __attribute__((always_inline)) {
    const int buf = c & 1, nt = min(C, N - c * C);
    const bf16_t *Kh = Kt[buf][0], *Kl = Kt[buf][1];
    const f32x4 z4{0.f, 0.f, 0.f, 0.f};
    load_tv(min(c + 1, nch - 1), tt2, rv2);  // past the end: reloads the last chunk (unused)
    // X = Kh W^T for token tile w; R = V - X (rows past the chunk are zero).
    {
      f32x4 X3[3] = {z4, z4, z4};
#pragma unroll
      for (int s = 0; s < SL; ++s)
        mma3s(unit16<U8>(Kh, 16 * w + n, 32 * s + 8 * g), unit16<U8>(Kl, 16 * w + n, 32 * s + 8 * g),
              unit16<U8>(Wt[buf][0], n, 32 * s + 8 * g), unit16<U8>(Wt[buf][1], n, 32 * s + 8 * g), X3);
      const f32x4 X = sum3(X3);
      f32x4 R;
#pragma unroll
      for (int r = 0; r < 4; ++r) R[r] = (16 * w + 4 * g + r < nt ? rv[r] : 0.f) - X[r];
      Rx[w][lane] = split4(R);
    }
    __syncthreads();
    // U = T R for token tile w.
    {
      f32x4 U3[3] = {z4, z4, z4};
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const bool on = sg == 0 || w >= 2;
        const u32x4 z{0u, 0u, 0u, 0u};
        const u32x4 a = Rx[2 * sg][lane], b = Rx[2 * sg + 1][lane];
        mma3s(on ? tt[2 * sg] : z, on ? tt[2 * sg + 1] : z, u32x4{a[0], a[1], b[0], b[1]},
              u32x4{a[2], a[3], b[2], b[3]}, U3);
      }
      Ux[w][lane] = split4(sum3(U3));
    }
    __syncthreads();
    // W^T tile dt += Kh^T U, and the memory after token tiles 0, 1, 2 (for the
    // outputs): slab 0 (tiles 0, 1), then slab 1 (tiles 2, 3); a tile alone is
    // the slab with the other tile's tokens zeroed in the Kh^T operand.
    {
      u32x4 uh[2], ul[2], ah[2], al[2];
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const u32x4 a = Ux[2 * sg][lane], b = Ux[2 * sg + 1][lane];
        uh[sg] = u32x4{a[0], a[1], b[0], b[1]};
        ul[sg] = u32x4{a[2], a[3], b[2], b[3]};
        ah[sg] = __builtin_bit_cast(u32x4, jfrag<U8>(Kh, 32 * sg, 16 * dt, g, n));
        al[sg] = __builtin_bit_cast(u32x4, jfrag<U8>(Kl, 32 * sg, 16 * dt, g, n));
      }
      const u32x4 lo2{0xffffffffu, 0xffffffffu, 0u, 0u};  // the first tile of a slab
      f32x4 A1[3] = {wm, z4, z4};
      mma3s(ah[0], al[0], uh[0], ul[0], A1);
      const f32x4 w1 = sum3(A1);  // after tiles 0, 1
      f32x4 F3[3] = {w1, z4, z4};
      mma3s(ah[1], al[1], uh[1], ul[1], F3);
      const f32x4 w0m = wm;
      wm = sum3(F3);  // the next chunk's memory
      put_w(Wt[buf ^ 1], wm);
      f32x4 A0[3] = {w0m, z4, z4}, A2[3] = {w1, z4, z4};
      mma3s(ah[0] & lo2, al[0] & lo2, uh[0], ul[0], A0);
      mma3s(ah[1] & lo2, al[1] & lo2, uh[1], ul[1], A2);
      put_w(Wp[0], sum3(A0));
      put_w(Wp[1], w1);
      put_w(Wp[2], sum3(A2));
    }
    __syncthreads();
  };

  // Helper waves.  Chunk c: the outputs of chunk c - 1; half of chunk c + 1
  // staged (kh copied, qh formed) and half of the q two chunks ahead loaded;
  // the other half, and the kh image two chunks ahead.  Past the last chunk the
  // staging writes zeros (no row is inside the chunk) into a buffer nothing
  // reads, and the loads re-read the last chunk: no branches.
  auto helper_chunk = [&](int c, float4 (&rq)[NU], u32x4 (&rk)[KU]) __attribute__((always_inline)) {
    const int buf = c & 1;
    const int cn = min(c + 2, nch - 1);
    outputs(c - 1);  // chunk 0: operands unused, nothing stored
    __syncthreads();
    copy_k(buf ^ 1, rk);
    stage_q(buf ^ 1, c + 1, rq, 0, NU / 2);
    load_q(cn, rq, 0, NU / 2);
    __syncthreads();
    stage_q(buf ^ 1, c + 1, rq, NU / 2, NU);
    load_q(cn, rq, NU / 2, NU);
    load_k(cn, rk);
    __syncthreads();
  };

  if (path) {
    u32x4 tta[4], ttb[4];
    float rva[4], rvb[4];
    load_tv(0, tta, rva);
    put_w(Wt[0], wm);
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
      path_chunk(c, tta, rva, ttb, rvb);
      if (c + 1 < nch) path_chunk(c + 1, ttb, rvb, tta, rva);
    }
    if (W_out && w < TD)
      *reinterpret_cast<float4*>(W_out + ((size_t)bh * M + m0 + n) * D + 16 * dt + 4 * g) =
          float4{wm[0], wm[1], wm[2], wm[3]};
  } else {
    float4 rq[NU];
    u32x4 rk[KU];
    load_q(0, rq, 0, NU);
    load_k(0, rk);
    copy_k(0, rk);
    stage_q(0, 0, rq, 0, NU);
    load_q(min(1, nch - 1), rq, 0, NU);
    load_k(min(1, nch - 1), rk);
    __syncthreads();
    for (int c = 0; c < nch; ++c) helper_chunk(c, rq, rk);
    outputs(nch - 1);
  }
}

// ----------------------------------------------------------------------------
// Host side.
template <typename T, int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, const void* beta, void* o, int BH, int N,
                       const float* W0, float* W_out, void* ws, hipStream_t stream) {
  const int nch = (N + C - 1) / C;
  u32x4* rec = (u32x4*)ws;
  hipLaunchKernelGGL((dn_prep_kernel<T, D>), dim3((unsigned)((size_t)BH * nch)), dim3(NT), 0, stream, (const T*)k,
                     (const T*)beta, N, nch, rec);
  const unsigned grid = (unsigned)(8 * ((BH + 7) / 8) * (M / 16));
  hipLaunchKernelGGL((dn_chain_kernel<T, D, M>), dim3(grid), dim3(NTC), 0, stream, (const T*)q, (const T*)v,
                     (const u32x4*)rec, BH, N, nch, W0, W_out, (T*)o);
  return hipGetLastError();
}

}  // namespace dnc

size_t deltanet_chunk_ws_bytes(int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0) return 0;
  if (!((D == 32 || D == 64) && (M == 32 || M == 64))) return 0;
  const size_t nch = (size_t)((N + dnc::C - 1) / dnc::C);
  const size_t units = D == 64 ? dnc::Rec<64>::UNITS : dnc::Rec<32>::UNITS;
  return (size_t)BH * nch * units * 16;
}

hipError_t launch_deltanet_chunked(const void* q, const void* k, const void* v, const void* beta, void* o, int BH,
                                   int N, int D, int M, int bf16, const float* W0, float* W_out, void* ws,
                                   hipStream_t stream) {
  if (bf16) {
    LA_DISPATCH_DM(dnc::impl, bf16_t, q, k, v, beta, o, BH, N, W0, W_out, ws, stream)
  } else {
    LA_DISPATCH_DM(dnc::impl, float, q, k, v, beta, o, BH, N, W0, W_out, ws, stream)
  }
}

}  // namespace la
