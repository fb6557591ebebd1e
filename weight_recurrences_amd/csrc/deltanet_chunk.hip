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
//   W_end = W0 + U^T Kh,   o_t = W0 qh_t + sum_{s<=t} (qh_t . kh_s) u_s.
// Only W0 -> W_end is sequential; it costs two small matrix products per chunk.
//
// Three kernels (fp32 arithmetic throughout, 16x16x4 f32 MFMA tiles):
//   dn_prep_kernel  per (head, chunk), in parallel: kh, G on MFMA, then Wc and Uc
//                   by forward substitution (one thread per column of [Kh | V]);
//                   writes Kh, Wc, Uc.
//   dn_scan_kernel  per (head, 16 rows of W): the chain over chunks,
//                   X = Wc W0^T (the slice's columns), U = Uc - X, W += U^T Kh;
//                   writes U and the memory at every chunk start.
//   dn_out_kernel   per (head, chunk), in parallel: o = Qh W0^T + (Qh Kh^T, j <= i) U.
//
// MFMA 16x16x4 f32 layouts (lane l = 16 g + n): operand a = A[n][g], b = B[g][n];
// the accumulator holds D[4g + r][n] in element r.  The k index of a product may
// be any permutation shared by both operands; the scan uses k = (tile dt, r) ->
// d = 16 dt + 4 g + r so that the transposed memory tiles it keeps in registers
// (the accumulator layout of the update) are directly the B operand of X.
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
  static constexpr size_t KH = (size_t)C * D, WC = (size_t)C * D, UC = (size_t)C * M, UU = (size_t)C * M,
                          WS = (size_t)M * D;
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
                                                     float* __restrict__ uc_ws) {
  using GG = G<D, M>;
  // Y = [Kh | V], one row per token: stride D + M + 4 keeps the column-slab reads
  // of the G product free of bank conflicts for every (D, M).
  constexpr int YS = D + M + 4;
  __shared__ __attribute__((aligned(16))) float Ys[C * YS];
  __shared__ __attribute__((aligned(16))) float Gs[C * GG::GS];
  __shared__ float Bs[C];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int t0 = c * C, nt = min(C, N - t0);
  float* Ks = Ys;  // kh: columns [0, D)
  load_rows<T, D, YS, true>(Ys, k + ((size_t)bh * N + t0) * D, nt, tid);
  load_rows<T, M, YS, false>(Ys + D, v + ((size_t)bh * N + t0) * M, nt, tid);
  if (tid < C) Bs[tid] = tid < nt ? ld_scalar<T>(beta + (size_t)bh * N + t0 + tid) : 0.f;
  __syncthreads();

  // G = Kh Kh^T: wave w computes the row tile w against every column tile.
#pragma unroll
  for (int jt = 0; jt < C / 16; ++jt) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Ks[(16 * w + n) * YS + 4 * kk + g], Ks[(16 * jt + n) * YS + 4 * kk + g], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Gs[(16 * w + 4 * g + r) * GG::GS + 16 * jt + n] = acc[r];
  }
  __syncthreads();

  // [Wc | Uc] = T [Kh | V]: x_t = beta_t (y_t - sum_{s<t} G[t][s] x_s), one column
  // per thread; the column stays in registers.
  const size_t rec = (size_t)bh * nch + c;
  if (tid < D + M) {
    float x[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
      float acc = Ys[t * YS + tid];
#pragma unroll
      for (int s = 0; s < t; ++s) acc -= Gs[t * GG::GS + s] * x[s];
      x[t] = Bs[t] * acc;
    }
    if (tid < D) {
#pragma unroll
      for (int t = 0; t < C; ++t) wc_ws[rec * GG::WC + (size_t)t * D + tid] = x[t];
    } else {
#pragma unroll
      for (int t = 0; t < C; ++t) uc_ws[rec * GG::UC + (size_t)t * M + (tid - D)] = x[t];
    }
  }
  // Kh for the scan and output kernels.
  float* khd = kh_ws + rec * GG::KH;
  for (int u = tid; u < C * D / 4; u += NT) {
    const int row = u / (D / 4), c4 = (u % (D / 4)) * 4;
    *reinterpret_cast<float4*>(&khd[row * D + c4]) = *reinterpret_cast<const float4*>(&Ks[row * YS + c4]);
  }
}

// ----------------------------------------------------------------------------
// Scan: grid (M/16) * BH, blockIdx.x = mg * BH + bh (the slices of one head are
// BH workgroups apart, so with BH a multiple of 8 they share an XCD and its L2).
// Wave w owns d-tile w of the transposed memory slice W^T[d][m0 .. m0 + 16); D/16
// of the 4 waves are used for the update, all 4 for X (one 16-token tile each).
template <int D, int M>
__global__ __launch_bounds__(NT) void dn_scan_kernel(const float* __restrict__ kh_ws, const float* __restrict__ wc_ws,
                                                     const float* __restrict__ uc_ws, const float* __restrict__ W0,
                                                     int BH, int nch, float* __restrict__ u_ws,
                                                     float* __restrict__ ws_ws, float* __restrict__ W_out) {
  using GG = G<D, M>;
  constexpr int WTS = C + 4;   // WcT row stride: (4g + r) * 68 = 16 g mod 64 banks
  constexpr int KHS = 80;      // kh row stride: (4kk + g) * 80 = 16 g mod 64 banks
  constexpr int UCS = 16;      // U / Uc slice row stride
  constexpr int TS = 20;       // W^T exchange row stride
  __shared__ __attribute__((aligned(16))) float WcT[D * WTS];  // Wc transposed: [d][t]
  __shared__ __attribute__((aligned(16))) float Khs[C * KHS];  // kh: [t][d]
  __shared__ __attribute__((aligned(16))) float Ucs[C * UCS];  // Uc slice: [t][m]
  __shared__ __attribute__((aligned(16))) float Us[C * UCS];   // U slice: [t][m]
  __shared__ __attribute__((aligned(16))) float Wts[D * TS];   // W^T slice: [d][m]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int mg = blockIdx.x / BH, bh = blockIdx.x % BH, m0 = 16 * mg;

  // wt[dt][r] = W^T[16 dt + 4 g + r][m0 + n]
  f32x4 wt[GG::TD];
#pragma unroll
  for (int dt = 0; dt < GG::TD; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wt[dt][r] = W0 ? W0[((size_t)bh * M + m0 + n) * D + 16 * dt + 4 * g + r] : 0.f;

  // Register staging of one chunk: Wc and kh as float4 units of rows, the Uc slice.
  constexpr int NW4 = C * D / 4 / NT;   // float4 units per thread (Wc and kh each)
  constexpr int NU4 = C * 16 / 4 / NT;  // Uc slice units per thread (1)
  float4 rw[NW4], rk[NW4], ru[NU4 > 0 ? NU4 : 1];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const size_t rec = (size_t)bh * nch + c;
#pragma unroll
    for (int i = 0; i < NW4; ++i) {
      const int u = tid + NT * i;
      rw[i] = *reinterpret_cast<const float4*>(wc_ws + rec * GG::WC + 4 * u);
      rk[i] = *reinterpret_cast<const float4*>(kh_ws + rec * GG::KH + 4 * u);
    }
#pragma unroll
    for (int i = 0; i < NU4; ++i) {
      const int u = tid + NT * i, row = u / 4, c4 = (u % 4) * 4;
      ru[i] = *reinterpret_cast<const float4*>(uc_ws + rec * GG::UC + (size_t)row * M + m0 + c4);
    }
  };
  load_chunk(0);

  for (int c = 0; c < nch; ++c) {
    const size_t rec = (size_t)bh * nch + c;
    // stage chunk c
#pragma unroll
    for (int i = 0; i < NW4; ++i) {
      const int u = tid + NT * i, row = u / (D / 4), c4 = (u % (D / 4)) * 4;
      WcT[(c4 + 0) * WTS + row] = rw[i].x;
      WcT[(c4 + 1) * WTS + row] = rw[i].y;
      WcT[(c4 + 2) * WTS + row] = rw[i].z;
      WcT[(c4 + 3) * WTS + row] = rw[i].w;
      *reinterpret_cast<float4*>(&Khs[row * KHS + c4]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < NU4; ++i) {
      const int u = tid + NT * i, row = u / 4, c4 = (u % 4) * 4;
      *reinterpret_cast<float4*>(&Ucs[row * UCS + c4]) = ru[i];
    }
    // the memory at the chunk start, for the output kernel (W layout [m][d])
    if (w < GG::TD)
      *reinterpret_cast<f32x4*>(ws_ws + rec * GG::WS + (size_t)(m0 + n) * D + 16 * w + 4 * g) = wt[w];
    __syncthreads();                     // (1) chunk staged
    if (c + 1 < nch) load_chunk(c + 1);  // in flight during the chain

    // X tile (tokens 16w .. 16w + 15) = Wc W0^T, k = (dt, r) -> d = 16 dt + 4 g + r
    f32x4 x{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = mma(WcT[(16 * dt + 4 * g + r) * WTS + 16 * w + n], wt[dt][r], x);
    // U = Uc - X: lane (n, g) holds rows t = 16w + 4g + r of column m0 + n
    f32x4 u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * g + r;
      u[r] = Ucs[t * UCS + n] - x[r];
      Us[t * UCS + n] = u[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) u_ws[rec * GG::UU + (size_t)(16 * w + 4 * g + r) * M + m0 + n] = u[r];
    __syncthreads();  // (2) U complete

    // W^T tile w += Kh^T U: A[d][t] = kh[t][d], B[t][m] = U[t][m]
    if (w < GG::TD) {
      f32x4 acc = wt[w];
#pragma unroll
      for (int kk = 0; kk < C / 4; ++kk) acc = mma(Khs[(4 * kk + g) * KHS + 16 * w + n], Us[(4 * kk + g) * UCS + n], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) Wts[(16 * w + 4 * g + r) * TS + n] = acc[r];
    }
    __syncthreads();  // (3) updated memory published
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wt[dt][r] = Wts[(16 * dt + 4 * g + r) * TS + n];
  }
  if (W_out && w < GG::TD)
    *reinterpret_cast<f32x4*>(W_out + ((size_t)bh * M + m0 + n) * D + 16 * w + 4 * g) = wt[w];
}

// ----------------------------------------------------------------------------
// Outputs: grid BH * nch, blockIdx.x = bh * nch + c.  Wave w owns tokens
// 16w .. 16w + 15 of the chunk.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void dn_out_kernel(const T* __restrict__ q, const float* __restrict__ kh_ws,
                                                    const float* __restrict__ u_ws, const float* __restrict__ ws_ws,
                                                    int N, int nch, T* __restrict__ o) {
  using GG = G<D, M>;
  __shared__ __attribute__((aligned(16))) float Qs[C * GG::KS];
  __shared__ __attribute__((aligned(16))) float Ks[C * GG::KS];
  __shared__ __attribute__((aligned(16))) float As[C * GG::GS];  // (qh . kh) with j <= i
  constexpr int US = M + 16;  // U row stride: (4kk + g) * US = 16 g mod 64 banks
  __shared__ __attribute__((aligned(16))) float Us[C * US];      // U [t][m]
  __shared__ __attribute__((aligned(16))) float Wss[M * GG::KS]; // W0 [m][d]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nch, c = blockIdx.x % nch;
  const int t0 = c * C, nt = min(C, N - t0);
  const size_t rec = (size_t)bh * nch + c;
  load_rows<T, D, GG::KS, true>(Qs, q + ((size_t)bh * N + t0) * D, nt, tid);
  load_rows<float, D, GG::KS, false>(Ks, kh_ws + rec * GG::KH, C, tid);
  load_rows<float, M, US, false>(Us, u_ws + rec * GG::UU, C, tid);
  load_rows<float, D, GG::KS, false, M>(Wss, ws_ws + rec * GG::WS, M, tid);
  __syncthreads();

  // A tiles of row tile w: (qh_i . kh_j), zero where j > i
#pragma unroll
  for (int st = 0; st < C / 16; ++st) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Qs[(16 * w + n) * GG::KS + 4 * kk + g], Ks[(16 * st + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * g + r, j = 16 * st + n;
      As[i * GG::GS + j] = j <= i ? acc[r] : 0.f;
    }
  }
  __syncthreads();

  T* oh = o + ((size_t)bh * N + t0) * M;
#pragma unroll
  for (int mt = 0; mt < GG::TM; ++mt) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk)
      acc = mma(Qs[(16 * w + n) * GG::KS + 4 * kk + g], Wss[(16 * mt + n) * GG::KS + 4 * kk + g], acc);
#pragma unroll
    for (int kk = 0; kk < C / 4; ++kk)
      acc = mma(As[(16 * w + n) * GG::GS + 4 * kk + g], Us[(4 * kk + g) * US + 16 * mt + n], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * g + r;
      if (t < nt) oh[(size_t)t * M + 16 * mt + n] = to_elem<T>(acc[r]);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
template <int D, int M>
static size_t ws_floats(int BH, int N) {
  using GG = G<D, M>;
  const size_t nch = (size_t)((N + C - 1) / C);
  return (size_t)BH * nch * (GG::KH + GG::WC + GG::UC + GG::UU + GG::WS);
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
  float* uu = uc + rec * GG::UC;
  float* wsb = uu + rec * GG::UU;
  const dim3 block(NT), grid((unsigned)rec);
  hipLaunchKernelGGL((dn_prep_kernel<T, D, M>), grid, block, 0, stream, (const T*)k, (const T*)v, (const T*)beta, N,
                     nch, kh, wc, uc);
  hipLaunchKernelGGL((dn_scan_kernel<D, M>), dim3((unsigned)(BH * (M / 16))), block, 0, stream, kh, wc, uc, W0, BH,
                     nch, uu, wsb, W_out);
  hipLaunchKernelGGL((dn_out_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, kh, uu, wsb, N, nch, (T*)o);
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
