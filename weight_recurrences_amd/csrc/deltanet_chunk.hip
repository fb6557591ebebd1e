// Chunk-parallel delta rule on gfx950.
//
// News summary of "Linear Transformers Are Secretly Fast Weight Programmers"
// (Schlag, Irie, Schmidhuber, 2021), paragraphs on the new update rule and on
// normalisation: per token, kh = phi(k)/sum phi(k), qh likewise,
// vbar = W kh, W += beta (v - vbar) kh^T, o = W qh (the updated memory).
//
// The same recurrence, regrouped by chunks of C = 64 tokens.  With W0 the memory
// at the chunk start and u_t = beta_t (v_t - W_{t-1} kh_t) the value actually
// written at token t, W_t = W0 + sum_{s<=t} u_s kh_s^T, so
//   u_t = beta_t (v_t - W0 kh_t - sum_{s<t} (kh_s . kh_t) u_s).
// This is a unit lower-triangular system in the rows u_t: with G = Kh Kh^T,
// L its strictly lower part and B = diag(beta), (I + B L) U = B (V - Kh W0^T),
// i.e. U = Uc - Wc W0^T with the memory-independent Wc = T Kh and Uc = T V,
// T = (I + B L)^{-1} B.  Then
//   W_end = W0 + U^T Kh = W0 A + Bc,  A = I - Wc^T Kh,  Bc = Uc^T Kh,
//   o_t = W0 qh_t + sum_{s<=t} (qh_t . kh_s) u_s.
// A chunk maps the memory by an affine map (A, Bc) that does not depend on it,
// so the only sequential work is one M x D by D x D product per chunk.
//
// Three kernels (fp32 arithmetic throughout, 16x16x4 f32 MFMA tiles):
//   dn_prep_kernel  per (head, chunk), in parallel: kh, G on MFMA, Wc and Uc by
//                   forward substitution (one thread per column of [Kh | V]),
//                   then A and Bc on MFMA; writes Kh, Wc, Uc, A, Bc.
//   dn_scan_kernel  per head: W <- W A + Bc over the chunks, each wave a
//                   16-row slice of W; writes the memory at every chunk start.
//                   Long sequences take two levels: dn_compose_kernel composes
//                   the maps of groups of 8 chunks in parallel, the scan runs
//                   over the composed maps, then over each group's chunks.
//   dn_out_kernel   per (head, chunk), in parallel: U = Uc - Wc W0^T, then
//                   o = Qh W0^T + (Qh Kh^T, j <= i) U.
//
// MFMA 16x16x4 f32 layouts (lane l = 16 g + n): operand a = A[n][g], b = B[g][n];
// the accumulator holds D[4g + r][n] in element r.  The k index of a product may
// be any permutation shared by both operands; the scan uses k = (tile dt, r) ->
// d = 16 dt + 4 g + r so that the transposed memory tiles it keeps in registers
// (its own accumulator layout) are directly the B operand of the next chunk.
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace dnc {

constexpr int NT = 256;  // threads per workgroup (4 wavefronts)
constexpr int C = 64;    // tokens per chunk

template <int D, int M>
struct G {
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int KS = D + 4;   // row stride of kh / qh tiles in LDS (floats)
  static constexpr int VS = M + 4;   // row stride of v tiles
  static constexpr int GS = C + 4;   // row stride of the C x C tiles
  // Per-chunk records in the workspace (floats).
  static constexpr size_t KH = (size_t)C * D, WC = (size_t)C * D, UC = (size_t)C * M, AA = (size_t)D * D,
                          BB = (size_t)M * D, WS = (size_t)M * D;
};

template <typename T> __device__ __forceinline__ float4 ld4(const T* p) { return load4<T>(p); }

// Loads ROWS rows of a [*, W] tensor (W = D or M) into an fp32 LDS tile with row
// stride S; with NORM, each row becomes phi(row) / sum(phi(row)).  Rows at or past
// nt are zero.  Thread p handles units of 4 elements.
template <typename T, int W, int S, bool NORM, int ROWS = C>
__device__ __forceinline__ void load_rows(float* tile, const T* src, int nt, int tid) {
  constexpr int UPR = W / 4;  // 4-element units per row
  constexpr int NU = ROWS * UPR;
#pragma unroll
  for (int i = 0; i < (NU + NT - 1) / NT; ++i) {
    const int u = tid + NT * i;
    if (NU % NT == 0 || u < NU) {  // uniform per group of UPR lanes
      const int row = u / UPR, c4 = (u % UPR) * 4;
      const bool ok = row < nt;
      float4 x = ok ? ld4<T>(src + (size_t)row * W + c4) : float4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NORM) {
        x = float4{phi(x.x), phi(x.y), phi(x.z), phi(x.w)};
        float s = (x.x + x.y) + (x.z + x.w);
        if constexpr (UPR == 16) s = sum16(s);
        else s = sum8(s);
        const float inv = ok ? 1.f / s : 0.f;
        x = float4{x.x * inv, x.y * inv, x.z * inv, x.w * inv};
      }
      *reinterpret_cast<float4*>(&tile[row * S + c4]) = x;
    }
  }
}

// ----------------------------------------------------------------------------
// Prep: grid BH * nch, blockIdx.x = bh * nch + c.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void dn_prep_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                     const T* __restrict__ beta, int N, int nch,
                                                     float* __restrict__ kh_ws, float* __restrict__ wc_ws,
                                                     float* __restrict__ uc_ws, float* __restrict__ a_ws,
                                                     float* __restrict__ b_ws) {
  using GG = G<D, M>;
  constexpr int W2 = D + M;       // columns of Y = [Kh | V] and of X = [Wc | Uc]
  constexpr int XS = W2 + 16;     // X row stride: rows read by k-slot g step 16 banks
  __shared__ __attribute__((aligned(16))) float Ks[C * GG::KS];  // Kh
  __shared__ __attribute__((aligned(16))) float Gs[C * GG::GS];  // G = Kh Kh^T
  __shared__ __attribute__((aligned(16))) float Xs[C * XS];      // Y, overwritten block by block by X
  __shared__ float Bs[C];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int t0 = c * C, nt = min(C, N - t0);
  load_rows<T, D, GG::KS, true>(Ks, k + ((size_t)bh * N + t0) * D, nt, tid);
  load_rows<T, M, XS, false>(Xs + D, v + ((size_t)bh * N + t0) * M, nt, tid);
  if (tid < C) Bs[tid] = tid < nt ? ld_scalar<T>(beta + (size_t)bh * N + t0 + tid) : 0.f;
  __syncthreads();
  for (int u = tid; u < C * D / 4; u += NT) {  // Y's Kh columns
    const int row = u / (D / 4), c4 = (u % (D / 4)) * 4;
    *reinterpret_cast<float4*>(&Xs[row * XS + c4]) = *reinterpret_cast<const float4*>(&Ks[row * GG::KS + c4]);
  }

  // G = Kh Kh^T: wave w computes the row tile w against every column tile.
#pragma unroll
  for (int jt = 0; jt < C / 16; ++jt) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Ks[(16 * w + n) * GG::KS + 4 * kk + g], Ks[(16 * jt + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Gs[(16 * w + 4 * g + r) * GG::GS + 16 * jt + n] = acc[r];
  }
  __syncthreads();

  // [Wc | Uc] = T [Kh | V], x_t = beta_t (y_t - sum_{s<t} G[t][s] x_s), in four
  // blocks of 16 tokens.  Block i first takes the earlier blocks at once on MFMA,
  // z = y - G[block i][blocks < i] X[blocks < i], in place in Xs; then one thread
  // per column solves the 16 rows of the block, right-looking (G is symmetric, so
  // column t of G is its row t).
#pragma unroll
  for (int bi = 0; bi < C / 16; ++bi) {
    if (bi > 0) {
      for (int ct = w; ct < W2 / 16; ct += 4) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Xs[(16 * bi + 4 * g + r) * XS + 16 * ct + n];
        for (int bj = 0; bj < bi; ++bj)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = mma(-Gs[(16 * bi + n) * GG::GS + 16 * bj + 4 * kk + g],
                      Xs[(16 * bj + 4 * kk + g) * XS + 16 * ct + n], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) Xs[(16 * bi + 4 * g + r) * XS + 16 * ct + n] = acc[r];
      }
      __syncthreads();
    }
    if (tid < W2) {
      float z[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) z[t] = Xs[(16 * bi + t) * XS + tid];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        z[t] *= Bs[16 * bi + t];
#pragma unroll
        for (int t2 = t + 1; t2 < 16; ++t2) z[t2] -= Gs[(16 * bi + t) * GG::GS + 16 * bi + t2] * z[t];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) Xs[(16 * bi + t) * XS + tid] = z[t];
    }
    __syncthreads();
  }

  const size_t rec = (size_t)bh * nch + c;
  // Wc, Uc and Kh for the output kernel.
  for (int u = tid; u < C * W2 / 4; u += NT) {
    const int row = u / (W2 / 4), c4 = (u % (W2 / 4)) * 4;
    const float4 x = *reinterpret_cast<const float4*>(&Xs[row * XS + c4]);
    if (c4 < D) *reinterpret_cast<float4*>(&wc_ws[rec * GG::WC + (size_t)row * D + c4]) = x;
    else *reinterpret_cast<float4*>(&uc_ws[rec * GG::UC + (size_t)row * M + c4 - D]) = x;
  }
  float* khd = kh_ws + rec * GG::KH;
  for (int u = tid; u < C * D / 4; u += NT) {
    const int row = u / (D / 4), c4 = (u % (D / 4)) * 4;
    *reinterpret_cast<float4*>(&khd[row * D + c4]) = *reinterpret_cast<const float4*>(&Ks[row * GG::KS + c4]);
  }

  // The chunk's affine map: A = I - Wc^T Kh (D x D), Bc = Uc^T Kh (M x D).  The
  // TD * TD + TM * TD output tiles are dealt round robin to the waves; tile
  // (i0, j0) = sum over tokens of X[t][i0 + i] Kh[t][j0 + j].
  constexpr int NTA = GG::TD * GG::TD, NTB = GG::TM * GG::TD;
  for (int tile = w; tile < NTA + NTB; tile += 4) {
    const bool isa = tile < NTA;
    const int tt = isa ? tile : tile - NTA;
    const int it = tt / GG::TD, jt = tt % GG::TD;
    const int xcol = (isa ? 0 : D) + 16 * it;
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C / 4; ++kk)
      acc = mma(Xs[(4 * kk + g) * XS + xcol + n], Ks[(4 * kk + g) * GG::KS + 16 * jt + n], acc);
    float* dst = isa ? a_ws + rec * GG::AA : b_ws + rec * GG::BB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * it + 4 * g + r, j = 16 * jt + n;
      dst[(size_t)i * D + j] = isa ? (i == j ? 1.f : 0.f) - acc[r] : acc[r];
    }
  }
}

// ----------------------------------------------------------------------------
// Scan: one workgroup per head; wave w keeps the 16-row slice m0 = 16 w of the
// memory, transposed, in registers: wt[dt][r] = W^T[16 dt + 4 g + r][m0 + n].
// Per chunk: W <- W A + Bc, i.e. W^T tile dt <- Bc^T tile dt + sum over k of
// A[k][16 dt + i] W^T[k][m], with k = 16 dt' + 4 g + r.  A (shared by the
// waves) is staged in LDS; each wave reads its Bc tiles from global memory.
// The workgroup covers the chunks [grp * G, min(nch, grp * G + G)) of head bh
// (blockIdx.x = bh * ng + grp, ng = ceil(nch / G)), starting from its own memory
// W0 + blockIdx.x * M * D; records are indexed bh * nch + c.  One workgroup per
// head (G = nch) is the plain scan.
template <int D, int M>
__global__ __launch_bounds__(NT) void dn_scan_kernel(const float* __restrict__ a_ws, const float* __restrict__ b_ws,
                                                     const float* __restrict__ W0, int nch, int G,
                                                     float* __restrict__ ws_ws, float* __restrict__ W_out) {
  using GG = dnc::G<D, M>;
  constexpr int AS = D + 4;  // A row stride: (4g + r) * AS = 16 g mod 64 banks at D = 64 (4 g at D = 32)
  __shared__ __attribute__((aligned(16))) float As[2][D * AS];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int ng = (nch + G - 1) / G, bh = blockIdx.x / ng, grp = blockIdx.x % ng, m0 = 16 * w;
  const int c0 = grp * G, c1 = min(nch, c0 + G);
  const bool active = w < GG::TM;  // waves past M/16 only help staging

  f32x4 wt[GG::TD];
#pragma unroll
  for (int dt = 0; dt < GG::TD; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wt[dt][r] = (W0 && active) ? W0[((size_t)blockIdx.x * M + m0 + n) * D + 16 * dt + 4 * g + r] : 0.f;

  // Register staging: A as float4 units of rows (all threads), this wave's Bc tiles.
  constexpr int NA4 = D * D / 4 / NT > 0 ? D * D / 4 / NT : 1;
  float4 ra[NA4];
  f32x4 rb[GG::TD];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const size_t rec = (size_t)bh * nch + c;
#pragma unroll
    for (int i = 0; i < NA4; ++i) {
      const int u = tid + NT * i;
      ra[i] = u < D * D / 4 ? *reinterpret_cast<const float4*>(a_ws + rec * GG::AA + 4 * u) : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt)
      rb[dt] = active ? *reinterpret_cast<const f32x4*>(b_ws + rec * GG::BB + (size_t)(m0 + n) * D + 16 * dt + 4 * g)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  load_chunk(c0);

  for (int c = c0; c < c1; ++c) {
    const size_t rec = (size_t)bh * nch + c;
    float* Ab = As[(c - c0) & 1];
#pragma unroll
    for (int i = 0; i < NA4; ++i) {
      const int u = tid + NT * i;
      if (u < D * D / 4) *reinterpret_cast<float4*>(&Ab[(u / (D / 4)) * AS + (u % (D / 4)) * 4]) = ra[i];
    }
    // the memory at the chunk start, for the output kernel (W layout [m][d])
    if (active) {
#pragma unroll
      for (int dt = 0; dt < GG::TD; ++dt)
        *reinterpret_cast<f32x4*>(ws_ws + rec * GG::WS + (size_t)(m0 + n) * D + 16 * dt + 4 * g) = wt[dt];
    }
    f32x4 acc[GG::TD];
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) acc[dt] = rb[dt];
    // One barrier per chunk: buffer c & 1 is rewritten two chunks later, after
    // every wave has passed the next chunk's barrier.
    __syncthreads();
    if (c + 1 < c1) load_chunk(c + 1);
#pragma unroll
    for (int dk = 0; dk < GG::TD; ++dk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < GG::TD; ++dt)
          acc[dt] = mma(Ab[(16 * dk + 4 * g + r) * AS + 16 * dt + n], wt[dk][r], acc[dt]);
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) wt[dt] = acc[dt];
  }
  if (W_out && active) {
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt)
      *reinterpret_cast<f32x4*>(W_out + ((size_t)blockIdx.x * M + m0 + n) * D + 16 * dt + 4 * g) = wt[dt];
  }
}

// ----------------------------------------------------------------------------
// Composition of the chunk maps of one group: W -> W A_c + Bc_c for the chunks
// [grp * G, min(nch, grp * G + G)) of head bh (blockIdx.x = bh * ng + grp) is
// W -> W Ag + Bg with (Ag, Bg) <- (Ag A_c, Bg A_c + Bc_c) from the group's first
// map.  Wave w holds rows 16 w.. of Ag (w < D / 16) and of Bg (w < M / 16) in the
// scan's transposed layout, so every step is the scan's product.  Writes
// ag [BH * ng][D][D] and bg [BH * ng][M][D].
template <int D, int M>
__global__ __launch_bounds__(NT) void dn_compose_kernel(const float* __restrict__ a_ws, const float* __restrict__ b_ws,
                                                        int nch, int G, float* __restrict__ ag, float* __restrict__ bg) {
  using GG = dnc::G<D, M>;
  constexpr int AS = D + 4;
  __shared__ __attribute__((aligned(16))) float As[2][D * AS];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int ng = (nch + G - 1) / G, bh = blockIdx.x / ng, grp = blockIdx.x % ng, r0 = 16 * w;
  const int c0 = grp * G, c1 = min(nch, c0 + G);
  const bool act_a = w < GG::TD, act_b = w < GG::TM;
  f32x4 xa[GG::TD], xb[GG::TD];
  {
    const size_t rec = (size_t)bh * nch + c0;
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      xa[dt] = act_a ? *reinterpret_cast<const f32x4*>(a_ws + rec * GG::AA + (size_t)(r0 + n) * D + 16 * dt + 4 * g)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
      xb[dt] = act_b ? *reinterpret_cast<const f32x4*>(b_ws + rec * GG::BB + (size_t)(r0 + n) * D + 16 * dt + 4 * g)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int c = c0 + 1; c < c1; ++c) {
    const size_t rec = (size_t)bh * nch + c;
    float* Ab = As[(c - c0) & 1];
    for (int u = tid; u < D * D / 4; u += NT)
      *reinterpret_cast<float4*>(&Ab[(u / (D / 4)) * AS + (u % (D / 4)) * 4]) =
          *reinterpret_cast<const float4*>(a_ws + rec * GG::AA + 4 * u);
    f32x4 acc_a[GG::TD], acc_b[GG::TD];
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      acc_a[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_b[dt] = act_b ? *reinterpret_cast<const f32x4*>(b_ws + rec * GG::BB + (size_t)(r0 + n) * D + 16 * dt + 4 * g)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // One barrier per chunk: buffer (c - c0) & 1 is rewritten two chunks later.
    __syncthreads();
#pragma unroll
    for (int dk = 0; dk < GG::TD; ++dk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < GG::TD; ++dt) {
          const float a = Ab[(16 * dk + 4 * g + r) * AS + 16 * dt + n];
          acc_a[dt] = mma(a, xa[dk][r], acc_a[dt]);
          acc_b[dt] = mma(a, xb[dk][r], acc_b[dt]);
        }
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      xa[dt] = acc_a[dt];
      xb[dt] = acc_b[dt];
    }
  }
#pragma unroll
  for (int dt = 0; dt < GG::TD; ++dt) {
    if (act_a)
      *reinterpret_cast<f32x4*>(ag + ((size_t)blockIdx.x * D + r0 + n) * D + 16 * dt + 4 * g) = xa[dt];
    if (act_b)
      *reinterpret_cast<f32x4*>(bg + ((size_t)blockIdx.x * M + r0 + n) * D + 16 * dt + 4 * g) = xb[dt];
  }
}

// ----------------------------------------------------------------------------
// Outputs: grid BH * nch, blockIdx.x = bh * nch + c.  Wave w owns tokens
// 16w .. 16w + 15 of the chunk.
//  1. U rows of the wave: U = Uc - Wc W0^T (in place over Uc in LDS).
//  2. Score tiles transposed, S^T[s][t] = kh_s . qh_t for the wave's tokens t,
//     zero where s > t.  Lane (n, g) of tile st holds s = 16 st + 4 g + r and
//     t = 16 w + n, which with k = (st, r) is exactly the A operand of step 3.
//  3. o = Qh W0^T + S U.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void dn_out_kernel(const T* __restrict__ q, const float* __restrict__ kh_ws,
                                                    const float* __restrict__ wc_ws, const float* __restrict__ uc_ws,
                                                    const float* __restrict__ ws_ws, int N, int nch,
                                                    T* __restrict__ o) {
  using GG = G<D, M>;
  constexpr int US = M + 4;  // U row stride: (4g + r) rows apart = 16 g mod 64 banks at M = 64
  __shared__ __attribute__((aligned(16))) float Xs[C * GG::KS];   // Wc rows, then qh rows
  __shared__ __attribute__((aligned(16))) float Ks[C * GG::KS];   // kh [t][d]
  __shared__ __attribute__((aligned(16))) float Wss[M * GG::KS];  // W0 [m][d]
  __shared__ __attribute__((aligned(16))) float Us[C * US];       // Uc, then U [t][m]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int t0 = c * C, nt = min(C, N - t0);
  const size_t rec = (size_t)bh * nch + c;
  load_rows<float, D, GG::KS, false>(Xs, wc_ws + rec * GG::WC, C, tid);
  load_rows<float, D, GG::KS, false>(Ks, kh_ws + rec * GG::KH, C, tid);
  load_rows<float, M, US, false>(Us, uc_ws + rec * GG::UC, C, tid);
  load_rows<float, D, GG::KS, false, M>(Wss, ws_ws + rec * GG::WS, M, tid);
  __syncthreads();

  // 1. U = Uc - Wc W0^T for tokens 16w .. 16w + 15
#pragma unroll
  for (int mt = 0; mt < GG::TM; ++mt) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Xs[(16 * w + n) * GG::KS + 4 * kk + g], Wss[(16 * mt + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float& u = Us[(16 * w + 4 * g + r) * US + 16 * mt + n];
      u = u - acc[r];
    }
  }
  __syncthreads();  // U complete; Wc no longer read
  load_rows<T, D, GG::KS, true>(Xs, q + ((size_t)bh * N + t0) * D, nt, tid);
  __syncthreads();

  // 2. transposed, masked score tiles
  f32x4 st4[C / 16];
#pragma unroll
  for (int st = 0; st < C / 16; ++st) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Ks[(16 * st + n) * GG::KS + 4 * kk + g], Xs[(16 * w + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (16 * st + 4 * g + r <= 16 * w + n) ? acc[r] : 0.f;
    st4[st] = acc;
  }

  // 3. o = Qh W0^T + S U
  T* oh = o + ((size_t)bh * N + t0) * M;
#pragma unroll
  for (int mt = 0; mt < GG::TM; ++mt) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Xs[(16 * w + n) * GG::KS + 4 * kk + g], Wss[(16 * mt + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int st = 0; st < C / 16; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mma(st4[st][r], Us[(16 * st + 4 * g + r) * US + 16 * mt + n], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * g + r;
      if (t < nt) oh[(size_t)t * M + 16 * mt + n] = to_elem<T>(acc[r]);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
// Chunks per group of the two-level scan (0: one serial scan per head).
static int scan_group(int nch) { return nch > 16 ? 8 : 0; }

template <int D, int M>
static size_t ws_floats(int BH, int N) {
  using GG = G<D, M>;
  const size_t nch = (size_t)((N + C - 1) / C);
  const int sg = scan_group((int)nch);
  const size_t ng = sg ? (nch + sg - 1) / sg : 0;
  // per chunk records, then per group: composed maps and the memory at the group start
  return (size_t)BH * nch * (GG::KH + GG::WC + GG::UC + GG::AA + GG::BB + GG::WS) +
         (size_t)BH * ng * (GG::AA + GG::BB + GG::WS);
}

template <typename T, int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, const void* beta, void* o, int BH, int N,
                       const float* W0, float* W_out, void* ws, hipStream_t stream) {
  using GG = G<D, M>;
  const int nch = (N + C - 1) / C;
  const size_t rec = (size_t)BH * nch;
  float* kh = (float*)ws;
  float* wc = kh + rec * GG::KH;
  float* uc = wc + rec * GG::WC;
  float* aa = uc + rec * GG::UC;
  float* bb = aa + rec * GG::AA;
  float* wsb = bb + rec * GG::BB;
  const dim3 block(NT), grid((unsigned)rec);
  hipLaunchKernelGGL((dn_prep_kernel<T, D, M>), grid, block, 0, stream, (const T*)k, (const T*)v, (const T*)beta, N,
                     nch, kh, wc, uc, aa, bb);
  const int sg = scan_group(nch);
  if (!sg) {
    hipLaunchKernelGGL((dn_scan_kernel<D, M>), dim3((unsigned)BH), block, 0, stream, aa, bb, W0, nch, nch, wsb, W_out);
  } else {
    // Two-level scan: the maps of each group of sg chunks are composed in
    // parallel, a short serial scan over the composed maps gives the memory at
    // every group start (and the final memory), and each group then replays its
    // own chunks from there in parallel, writing the memory at every chunk start.
    const int ng = (nch + sg - 1) / sg;
    float* ag = wsb + rec * GG::WS;
    float* bg = ag + (size_t)BH * ng * GG::AA;
    float* wg = bg + (size_t)BH * ng * GG::BB;
    hipLaunchKernelGGL((dn_compose_kernel<D, M>), dim3((unsigned)(BH * ng)), block, 0, stream, aa, bb, nch, sg, ag, bg);
    hipLaunchKernelGGL((dn_scan_kernel<D, M>), dim3((unsigned)BH), block, 0, stream, ag, bg, W0, ng, ng, wg, W_out);
    hipLaunchKernelGGL((dn_scan_kernel<D, M>), dim3((unsigned)(BH * ng)), block, 0, stream, aa, bb, wg, nch, sg, wsb,
                       nullptr);
  }
  hipLaunchKernelGGL((dn_out_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, kh, wc, uc, wsb, N, nch, (T*)o);
  return hipGetLastError();
}

}  // namespace dnc

size_t deltanet_chunk_ws_bytes(int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0) return 0;
  switch (D * 100 + M) {
    case 3232: return dnc::ws_floats<32, 32>(BH, N) * sizeof(float);
    case 3264: return dnc::ws_floats<32, 64>(BH, N) * sizeof(float);
    case 6432: return dnc::ws_floats<64, 32>(BH, N) * sizeof(float);
    case 6464: return dnc::ws_floats<64, 64>(BH, N) * sizeof(float);
    default: return 0;
  }
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
