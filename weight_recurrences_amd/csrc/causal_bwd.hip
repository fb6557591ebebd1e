// Backward of causal linear attention on gfx950: the float32 path (fp32 MFMA);
// bf16 inputs take the bf16 MFMA kernels of causal_bwd_bf16.hip after the
// shared block-prefix step.
//
// "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.3 eq.(9)-(12) and §3.3.1: the gradients of the causal form
// are cumulative sums, computed in linear time with constant memory per state.
// The page omits the equations; they follow from eq.(9)-(12).  With
// num_i = S_i^T phi(q_i), den_i = z_i . phi(q_i), o_i = num_i / den_i and the
// loss gradient dO_i,
//   a_i = dO_i / den_i,                b_i = -(dO_i . num_i) / den_i^2,
//   dphi(q_i) = S_i a_i + z_i b_i                       (a prefix sum, as eq.(10)-(11))
//   dphi(k_j) = sum_{i>=j} phi(q_i) (a_i . v_j + b_i)   (a suffix sum)
//   dv_j      = sum_{i>=j} (phi(q_i) . phi(k_j)) a_i
// and dq = dphi(q) * phi'(q), phi'(x) = 1 (x > 0), e^x otherwise = min(phi(x), 1).
//
// Chunks of C = 64 tokens, with P = tril(phi(Q) phi(K)^T) and
// E = tril(a V^T + b 1^T) (j <= i inclusive):
//   forward sweep:  dphi(Q) = a S^T + b z^T + E phi(K),  then S += phi(K)^T V, z += colsum phi(K)
//   reverse sweep:  dphi(K) = V R^T + 1 r^T + E^T phi(Q),  dV = phi(K) R + P^T a,
//                   then R += phi(Q)^T a, r += phi(Q)^T b
// where (S, z) is the prefix state before the chunk and (R, r) the suffix state
// after it.  Blocks of T tokens fill the GPU: the prefix states of the blocks
// come from the forward pass's block kernels and scan; the suffix states from
// the per-block sums of phi(Q)^T a and phi(Q)^T b and a reverse scan.
//
// Kernels:
//   bwd_q_kernel       forward sweep per block: a, b (kept in the workspace) and dq
//   bwd_rstate_kernel  per block: sum of phi(q_i) a_i^T and phi(q_i) b_i
//   suffix_scan_kernel per head: exclusive suffix sums of those block sums
//   bwd_kv_kernel      reverse sweep per block: dk, dv
//
// MFMA 16x16x4 f32 (lane l = 16 g + n): a = A[n][g], b = B[g][n], the
// accumulator holds D[4g + r][n].  Wave w owns the 16 rows 16w .. 16w + 15 of
// each chunk; products are formed transposed (rows = feature, columns = token)
// so that a tile computed in registers is directly the operand of the next
// product under the k permutation k = 16 t + 4 g + r.
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace bwd {

constexpr int NT = 256;
constexpr int C = 64;

template <int D, int M>
struct G {
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int SD = D + 4, SM = M + 4;  // LDS row strides (floats)
  static constexpr int SZ = D * M + D;          // floats of an (S, z) record
};

// Token rows [0, C) of a [*, W] tensor into an fp32 LDS tile (row stride S):
// plain, or phi applied; rows at or past nt are zero.
template <typename T, int W, int S, bool PHI>
__device__ __forceinline__ void load_tile(float* tile, const T* src, int nt, int tid) {
  constexpr int UPR = W / 4, NU = C * UPR;
#pragma unroll
  for (int i = 0; i < NU / NT; ++i) {
    const int u = tid + NT * i, row = u / UPR, c4 = (u % UPR) * 4;
    float4 x = row < nt ? load4<T>(src + (size_t)row * W + c4) : float4{0.f, 0.f, 0.f, 0.f};
    if (PHI && row < nt) x = float4{phi(x.x), phi(x.y), phi(x.z), phi(x.w)};
    *reinterpret_cast<float4*>(&tile[row * S + c4]) = x;
  }
}

__device__ __forceinline__ float dphi_of(float ph) { return fminf(ph, 1.f); }  // phi' from phi

// ----------------------------------------------------------------------------
// Forward sweep.  Grid BH * nblk; the block's prefix state is (preS, preZ).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void bwd_q_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const T* __restrict__ dO,
                                                   T* __restrict__ dq, int N, int tblk, int nblk,
                                                   const float* __restrict__ preS, const float* __restrict__ preZ,
                                                   float* __restrict__ a_ws, float* __restrict__ b_ws) {
  using GG = G<D, M>;
  constexpr int SD = GG::SD, SM = GG::SM;
  __shared__ __attribute__((aligned(16))) float Qs[C * SD];  // phi(q)
  __shared__ __attribute__((aligned(16))) float Ks[C * SD];  // phi(k)
  __shared__ __attribute__((aligned(16))) float Vs[C * SM];
  __shared__ __attribute__((aligned(16))) float Gs[C * SM];  // dO
  __shared__ __attribute__((aligned(16))) float Ss[D * SM];  // S [d][m]
  __shared__ float Zs[D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  {
    const size_t rec = (size_t)bh * nblk + blk;
    for (int e = tid; e < D * M; e += NT) Ss[(e / M) * SM + e % M] = preS[rec * D * M + e];
    if (tid < D) Zs[tid] = preZ[rec * D + tid];
  }
  const int i_loc = 16 * w + n;

  for (int c0 = t0; c0 < t1; c0 += C) {
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();  // the previous chunk's readers and state update are done
    load_tile<T, D, SD, true>(Qs, q + row0 * D, nt, tid);
    load_tile<T, D, SD, true>(Ks, k + row0 * D, nt, tid);
    load_tile<T, M, SM, false>(Vs, v + row0 * M, nt, tid);
    load_tile<T, M, SM, false>(Gs, dO + row0 * M, nt, tid);
    __syncthreads();

    // (1) PT[jt][r] = P[i][j], i = 16w + n, j = 16 jt + 4g + r, zero where j > i
    f32x4 PT[C / 16];
#pragma unroll
    for (int jt = 0; jt < C / 16; ++jt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk)
        acc = mma(Ks[(16 * jt + n) * SD + 4 * kk + g], Qs[i_loc * SD + 4 * kk + g], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (16 * jt + 4 * g + r <= i_loc) ? acc[r] : 0.f;
      PT[jt] = acc;
    }
    // (2) numT[mt][r] = num[i][m], m = 16 mt + 4g + r:  S^T phi(q_i) + sum_j P[i][j] v_j
    f32x4 numT[GG::TM];
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk)
        acc = mma(Ss[(4 * kk + g) * SM + 16 * mt + n], Qs[i_loc * SD + 4 * kk + g], acc);
#pragma unroll
      for (int jt = 0; jt < C / 16; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(Vs[(16 * jt + 4 * g + r) * SM + 16 * mt + n], PT[jt][r], acc);
      numT[mt] = acc;
    }
    // (3) den_i = z . phi(q_i) + sum_j P[i][j] (every element of the tile)
    float den;
    {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk) acc = mma(Zs[4 * kk + g], Qs[i_loc * SD + 4 * kk + g], acc);
#pragma unroll
      for (int jt = 0; jt < C / 16; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(1.f, PT[jt][r], acc);
      den = acc[0];
    }
    // (4) a_i = dO_i / den_i, b_i = -(dO_i . num_i) / den_i^2
    const bool rowok = i_loc < nt;
    const float inv = rowok ? 1.f / den : 0.f;
    f32x4 aT[GG::TM];
    float bp = 0.f;
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      const f32x4 go = *reinterpret_cast<const f32x4*>(&Gs[i_loc * SM + 16 * mt + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        aT[mt][r] = go[r] * inv;
        bp += go[r] * numT[mt][r];
      }
    }
    bp += __shfl_xor(bp, 16);
    bp += __shfl_xor(bp, 32);
    const float b = -bp * inv * inv;
    if (rowok) {
#pragma unroll
      for (int mt = 0; mt < GG::TM; ++mt)
        *reinterpret_cast<f32x4*>(a_ws + (row0 + i_loc) * M + 16 * mt + 4 * g) = aT[mt];
      if (g == 0) b_ws[row0 + i_loc] = b;
    }
    // (5) ET[jt][r] = E[i][j] = a_i . v_j + b_i, zero where j > i
    f32x4 ET[C / 16];
#pragma unroll
    for (int jt = 0; jt < C / 16; ++jt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < GG::TM; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(Vs[(16 * jt + n) * SM + 16 * mt + 4 * g + r], aT[mt][r], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (16 * jt + 4 * g + r <= i_loc) ? acc[r] + b : 0.f;
      ET[jt] = acc;
    }
    // (6) dphi(q_i)[d] = (S a_i)[d] + z[d] b_i + sum_j E[i][j] phi(k_j)[d];  dq = dphi(q) * phi'(q)
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < GG::TM; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(Ss[(16 * dt + n) * SM + 16 * mt + 4 * g + r], aT[mt][r], acc);
#pragma unroll
      for (int jt = 0; jt < C / 16; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(Ks[(16 * jt + 4 * g + r) * SD + 16 * dt + n], ET[jt][r], acc);
      float4 out;
      const f32x4 fq = *reinterpret_cast<const f32x4*>(&Qs[i_loc * SD + 16 * dt + 4 * g]);
      out.x = (acc[0] + Zs[16 * dt + 4 * g + 0] * b) * dphi_of(fq[0]);
      out.y = (acc[1] + Zs[16 * dt + 4 * g + 1] * b) * dphi_of(fq[1]);
      out.z = (acc[2] + Zs[16 * dt + 4 * g + 2] * b) * dphi_of(fq[2]);
      out.w = (acc[3] + Zs[16 * dt + 4 * g + 3] * b) * dphi_of(fq[3]);
      if (rowok) store4<T>(dq + (row0 + i_loc) * D + 16 * dt + 4 * g, out);
    }
    __syncthreads();  // every read of S and z is done

    // (7) S += phi(K)^T V, z += colsum phi(K); wave w updates d-tiles w, w + 4, ...
    for (int dt = w; dt < GG::TD; dt += 4) {
#pragma unroll
      for (int mt = 0; mt < GG::TM; ++mt) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Ss[(16 * dt + 4 * g + r) * SM + 16 * mt + n];
#pragma unroll
        for (int kk = 0; kk < C / 4; ++kk)
          acc = mma(Ks[(4 * kk + g) * SD + 16 * dt + n], Vs[(4 * kk + g) * SM + 16 * mt + n], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[(16 * dt + 4 * g + r) * SM + 16 * mt + n] = acc[r];
      }
      f32x4 zc;
#pragma unroll
      for (int r = 0; r < 4; ++r) zc[r] = Zs[16 * dt + 4 * g + r];
#pragma unroll
      for (int kk = 0; kk < C / 4; ++kk) zc = mma(Ks[(4 * kk + g) * SD + 16 * dt + n], 1.f, zc);
      if (n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Zs[16 * dt + 4 * g + r] = zc[r];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Per-block suffix contributions: R_b = sum_{i in b} phi(q_i) a_i^T [D][M],
// r_b = sum_{i in b} phi(q_i) b_i [D], into suf[bh][blk] (SZ floats).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void bwd_rstate_kernel(const T* __restrict__ q, const float* __restrict__ a_ws,
                                                        const float* __restrict__ b_ws, int N, int tblk, int nblk,
                                                        float* __restrict__ suf) {
  using GG = G<D, M>;
  constexpr int SD = GG::SD, SM = GG::SM;
  __shared__ __attribute__((aligned(16))) float Qs[C * SD];
  __shared__ __attribute__((aligned(16))) float As[C * SM];
  __shared__ float Bs[C];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const int dt = w;  // waves w < D/16 own d-tile w
  f32x4 R[GG::TM], rz{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < GG::TM; ++mt) R[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = t0; c0 < t1; c0 += C) {
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();
    load_tile<T, D, SD, true>(Qs, q + row0 * D, nt, tid);
    load_tile<float, M, SM, false>(As, a_ws + row0 * M, nt, tid);
    if (tid < C) Bs[tid] = tid < nt ? b_ws[row0 + tid] : 0.f;
    __syncthreads();
    if (dt < GG::TD) {
#pragma unroll
      for (int kk = 0; kk < C / 4; ++kk) {
        const float a = Qs[(4 * kk + g) * SD + 16 * dt + n];
#pragma unroll
        for (int mt = 0; mt < GG::TM; ++mt) R[mt] = mma(a, As[(4 * kk + g) * SM + 16 * mt + n], R[mt]);
        rz = mma(a, Bs[4 * kk + g], rz);
      }
    }
  }
  if (dt < GG::TD) {
    float* dst = suf + ((size_t)bh * nblk + blk) * GG::SZ;
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * dt + 4 * g + r) * M + 16 * mt + n] = R[mt][r];
    if (n == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[D * M + 16 * dt + 4 * g + r] = rz[r];
    }
  }
}

// Exclusive suffix sums over the blocks of each head, in place:
// suf[b] <- sum_{b' > b} suf[b'] (fixed order, bitwise repeatable).
__global__ __launch_bounds__(NT) void suffix_scan_kernel(float* suf, int nblk, int SZ) {
  const int parts = (SZ + NT - 1) / NT;
  const int e = (blockIdx.x % parts) * NT + threadIdx.x, bh = blockIdx.x / parts;
  if (e >= SZ) return;
  float* base = suf + (size_t)bh * nblk * SZ + e;
  float run = 0.f;
  for (int b = nblk - 1; b >= 0; --b) {
    const float t = base[(size_t)b * SZ];
    base[(size_t)b * SZ] = run;
    run += t;
  }
}

// ----------------------------------------------------------------------------
// Reverse sweep.  Grid BH * nblk; the block's suffix state is suf[bh][blk].
// Chunks run from the last to the first; wave w owns key rows j = 16w + n.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void bwd_kv_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ a_ws,
                                                    const float* __restrict__ b_ws, T* __restrict__ dk,
                                                    T* __restrict__ dv, int N, int tblk, int nblk,
                                                    const float* __restrict__ suf) {
  using GG = G<D, M>;
  constexpr int SD = GG::SD, SM = GG::SM;
  __shared__ __attribute__((aligned(16))) float Qs[C * SD];
  __shared__ __attribute__((aligned(16))) float Ks[C * SD];
  __shared__ __attribute__((aligned(16))) float Vs[C * SM];
  __shared__ __attribute__((aligned(16))) float As[C * SM];
  __shared__ __attribute__((aligned(16))) float Rs[D * SM];  // R [d][m]
  __shared__ float Bs[C];
  __shared__ float rs[D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  {
    const float* src = suf + ((size_t)bh * nblk + blk) * GG::SZ;
    for (int e = tid; e < D * M; e += NT) Rs[(e / M) * SM + e % M] = src[e];
    if (tid < D) rs[tid] = src[D * M + tid];
  }
  const int j_loc = 16 * w + n;
  const int nchb = (t1 - t0 + C - 1) / C;

  for (int ci = nchb - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * C;
    const int nt = min(C, t1 - c0);
    const size_t row0 = (size_t)bh * N + c0;
    __syncthreads();
    load_tile<T, D, SD, true>(Qs, q + row0 * D, nt, tid);
    load_tile<T, D, SD, true>(Ks, k + row0 * D, nt, tid);
    load_tile<T, M, SM, false>(Vs, v + row0 * M, nt, tid);
    load_tile<float, M, SM, false>(As, a_ws + row0 * M, nt, tid);
    if (tid < C) Bs[tid] = tid < nt ? b_ws[row0 + tid] : 0.f;
    __syncthreads();

    // (1) PJ[it][r] = P[i][j], i = 16 it + 4g + r, j = 16w + n, zero where i < j
    // (2) EJ[it][r] = E[i][j] = a_i . v_j + b_i, zero where i < j
    f32x4 PJ[C / 16], EJ[C / 16];
#pragma unroll
    for (int it = 0; it < C / 16; ++it) {
      f32x4 p{0.f, 0.f, 0.f, 0.f}, e{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk)
        p = mma(Qs[(16 * it + n) * SD + 4 * kk + g], Ks[j_loc * SD + 4 * kk + g], p);
#pragma unroll
      for (int kk = 0; kk < M / 4; ++kk)
        e = mma(As[(16 * it + n) * SM + 4 * kk + g], Vs[j_loc * SM + 4 * kk + g], e);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g + r;
        p[r] = i >= j_loc ? p[r] : 0.f;
        e[r] = i >= j_loc ? e[r] + Bs[i] : 0.f;
      }
      PJ[it] = p;
      EJ[it] = e;
    }
    const bool rowok = j_loc < nt;
    // (3) dv_j[m] = (R^T phi(k_j))[m] + sum_i P[i][j] a_i[m]
#pragma unroll
    for (int mt = 0; mt < GG::TM; ++mt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk)
        acc = mma(Rs[(4 * kk + g) * SM + 16 * mt + n], Ks[j_loc * SD + 4 * kk + g], acc);
#pragma unroll
      for (int it = 0; it < C / 16; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(As[(16 * it + 4 * g + r) * SM + 16 * mt + n], PJ[it][r], acc);
      if (rowok) store4<T>(dv + (row0 + j_loc) * M + 16 * mt + 4 * g, float4{acc[0], acc[1], acc[2], acc[3]});
    }
    // (4) dphi(k_j)[d] = (R v_j)[d] + r[d] + sum_i E[i][j] phi(q_i)[d];  dk = dphi(k) * phi'(k)
#pragma unroll
    for (int dt = 0; dt < GG::TD; ++dt) {
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < M / 4; ++kk)
        acc = mma(Rs[(16 * dt + n) * SM + 4 * kk + g], Vs[j_loc * SM + 4 * kk + g], acc);
#pragma unroll
      for (int it = 0; it < C / 16; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mma(Qs[(16 * it + 4 * g + r) * SD + 16 * dt + n], EJ[it][r], acc);
      const f32x4 fk = *reinterpret_cast<const f32x4*>(&Ks[j_loc * SD + 16 * dt + 4 * g]);
      float4 out;
      out.x = (acc[0] + rs[16 * dt + 4 * g + 0]) * dphi_of(fk[0]);
      out.y = (acc[1] + rs[16 * dt + 4 * g + 1]) * dphi_of(fk[1]);
      out.z = (acc[2] + rs[16 * dt + 4 * g + 2]) * dphi_of(fk[2]);
      out.w = (acc[3] + rs[16 * dt + 4 * g + 3]) * dphi_of(fk[3]);
      if (rowok) store4<T>(dk + (row0 + j_loc) * D + 16 * dt + 4 * g, out);
    }
    __syncthreads();  // every read of R and r is done

    // (5) R += phi(Q)^T a, r += phi(Q)^T b; wave w updates d-tiles w, w + 4, ...
    for (int dt = w; dt < GG::TD; dt += 4) {
#pragma unroll
      for (int mt = 0; mt < GG::TM; ++mt) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Rs[(16 * dt + 4 * g + r) * SM + 16 * mt + n];
#pragma unroll
        for (int kk = 0; kk < C / 4; ++kk)
          acc = mma(Qs[(4 * kk + g) * SD + 16 * dt + n], As[(4 * kk + g) * SM + 16 * mt + n], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) Rs[(16 * dt + 4 * g + r) * SM + 16 * mt + n] = acc[r];
      }
      f32x4 rc;
#pragma unroll
      for (int r = 0; r < 4; ++r) rc[r] = rs[16 * dt + 4 * g + r];
#pragma unroll
      for (int kk = 0; kk < C / 4; ++kk) rc = mma(Qs[(4 * kk + g) * SD + 16 * dt + n], Bs[4 * kk + g], rc);
      if (n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[16 * dt + 4 * g + r] = rc[r];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
template <int D, int M>
struct Layout {
  size_t preS, preZ, a, b, suf, total;  // float offsets
  Layout(int BH, int N, int nblk) {
    preS = 0;
    preZ = preS + (size_t)BH * nblk * D * M;
    a = preZ + (size_t)BH * nblk * D;
    a = (a + 3) / 4 * 4;  // 16-byte alignment of the a rows
    b = a + (size_t)BH * N * M;
    suf = b + (size_t)BH * N;
    suf = (suf + 3) / 4 * 4;
    total = suf + (size_t)BH * nblk * G<D, M>::SZ;
  }
};

// Block length of the backward: the sweeps are chains of dependent chunks, and
// one round of resident workgroups (two per CU, 512 in all) runs faster than two
// rounds of half the length (long workload: 604.6 us per call with 2048-token
// blocks, 632.0 with 1024, 644.2 with 512).
static int bwd_block_tokens(int BH, int N) {
  if (N <= 0 || BH <= 0) return 64;
  const int per_head = BH >= 512 ? 1 : (512 + BH - 1) / BH;
  int tb = (N + per_head - 1) / per_head;
  tb = ((tb + 63) / 64) * 64;
  if (tb < 256) tb = 256;
  const int ncap = ((N + 63) / 64) * 64;
  if (tb > ncap) tb = ncap;
  return tb;
}

template <int D, int M>
static size_t ws_bytes(int BH, int N) {
  const int tblk = bwd_block_tokens(BH, N);
  const int nblk = (N + tblk - 1) / tblk;
  return Layout<D, M>(BH, N, nblk).total * sizeof(float);
}

template <typename T, int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk, void* dv,
                       int BH, int N, void* ws, hipStream_t stream) {
  using GG = G<D, M>;
  const int tblk = bwd_block_tokens(BH, N);
  const int nblk = (N + tblk - 1) / tblk;
  const Layout<D, M> l(BH, N, nblk);
  float* base = (float*)ws;
  float *preS = base + l.preS, *preZ = base + l.preZ, *aw = base + l.a, *bw = base + l.b, *suf = base + l.suf;
  hipError_t e = launch_block_prefix(k, v, BH, N, D, M, sizeof(T) == 2, tblk, nblk, preS, preZ, stream);
  if (e != hipSuccess) return e;
  if constexpr (sizeof(T) == 2)  // bf16 MFMA kernels; 1/den in the first BH * N floats of the a region
    return launch_causal_bwd_bf16(q, k, v, dO, dq, dk, dv, BH, N, D, M, tblk, nblk, preS, preZ, aw, bw, suf, stream);
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(NT);
  hipLaunchKernelGGL((bwd_q_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, (const T*)k, (const T*)v,
                     (const T*)dO, (T*)dq, N, tblk, nblk, preS, preZ, aw, bw);
  hipLaunchKernelGGL((bwd_rstate_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, aw, bw, N, tblk, nblk, suf);
  const int parts = (GG::SZ + NT - 1) / NT;
  hipLaunchKernelGGL(suffix_scan_kernel, dim3((unsigned)(parts * BH)), block, 0, stream, suf, nblk, GG::SZ);
  hipLaunchKernelGGL((bwd_kv_kernel<T, D, M>), grid, block, 0, stream, (const T*)q, (const T*)k, (const T*)v, aw, bw,
                     (T*)dk, (T*)dv, N, tblk, nblk, suf);
  return hipGetLastError();
}

}  // namespace bwd

hipError_t launch_suffix_scan(float* suf, int BH, int nblk, int SZ, hipStream_t stream) {
  const int parts = (SZ + bwd::NT - 1) / bwd::NT;
  hipLaunchKernelGGL(bwd::suffix_scan_kernel, dim3((unsigned)(parts * BH)), dim3(bwd::NT), 0, stream, suf, nblk, SZ);
  return hipGetLastError();
}

size_t causal_bwd_ws_bytes(int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0) return 0;
  switch (D * 100 + M) {
    case 3232: return bwd::ws_bytes<32, 32>(BH, N);
    case 3264: return bwd::ws_bytes<32, 64>(BH, N);
    case 6432: return bwd::ws_bytes<64, 32>(BH, N);
    case 6464: return bwd::ws_bytes<64, 64>(BH, N);
    default: return 0;
  }
}

hipError_t launch_causal_bwd(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk,
                             void* dv, int BH, int N, int D, int M, int bf16, void* ws, hipStream_t stream) {
  if (BH == 0 || N == 0) return hipSuccess;
  if (bf16) {
    LA_DISPATCH_DM(bwd::impl, bf16_t, q, k, v, dO, dq, dk, dv, BH, N, ws, stream)
  } else {
    LA_DISPATCH_DM(bwd::impl, float, q, k, v, dO, dq, dk, dv, BH, N, ws, stream)
  }
}

}  // namespace la
