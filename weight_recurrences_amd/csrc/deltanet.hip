// Delta-rule fast-weight memory on gfx950.
//
// News summary of "Linear Transformers Are Secretly Fast Weight Programmers"
// (Schlag, Irie, Schmidhuber, 2021), paragraphs on the new update rule and on
// normalisation: for each token, retrieve the value currently bound to the
// key, vbar = W kh, and replace it by the convex combination
// beta v + (1 - beta) vbar, i.e. W += beta (v - vbar) kh^T; keys and queries
// pass through phi = elu + 1 and are divided by the sum of their components;
// the output reads the updated memory, o = W qh.
//
// Rows of W are independent chains (row m only ever sees v_m), so the memory of
// a (b, h) is split over workgroups of 16 rows: 4 wavefronts x 4 rows, 16
// lanes per row, D/16 consecutive elements of the row per lane, all in
// registers.  The token loop is inherently sequential; what does not depend on
// W (phi, the sum normalisation of k and q, the loads) is computed for a block
// of 64 tokens at a time by the whole workgroup and staged in LDS, with the
// next block's global loads in flight during the sequential phase.
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "kernels.hpp"

namespace la {

constexpr int DTB = 64;  // tokens per staged block

template <typename T, int D, int M>
__global__ __launch_bounds__(256) void deltanet_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const T* __restrict__ beta,
                                                       T* __restrict__ o, int N, const float* W0, float* W_out) {
  constexpr int DPL = D / 16;   // elements of a row per lane
  constexpr int UPT = D / 4;    // 4-element units per token row of k/q
  constexpr int NU = DTB * UPT; // units per block
  constexpr int KU = (NU + 255) / 256;
  __shared__ __attribute__((aligned(16))) float Kh[DTB][D + 4];
  __shared__ __attribute__((aligned(16))) float Qh[DTB][D + 4];
  __shared__ __attribute__((aligned(16))) float Vs[DTB][16];
  __shared__ float Bs[DTB];
  __shared__ float Os[DTB][17];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, rl = lane >> 4;
  const int rg = blockIdx.x % (M / 16), bh = blockIdx.x / (M / 16);
  const int m = 16 * rg + 4 * w + rl;  // memory row owned by this lane group

  const T* qh = q + (size_t)bh * N * D;
  const T* kh = k + (size_t)bh * N * D;
  const T* vh = v + (size_t)bh * N * M;
  const T* bhp = beta + (size_t)bh * N;
  T* oh = o + (size_t)bh * N * M;

  float W[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) W[e] = W0 ? W0[((size_t)bh * M + m) * D + n * DPL + e] : 0.f;

  // Register prefetch of one block: k, q units, one v unit, one beta.
  float4 rk[KU], rq[KU], rv;
  float rb;
  auto prefetch = [&](int t0, int nt) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + 256 * i;
      const int tok = u / UPT, d4 = (u % UPT) * 4;
      rk[i] = rq[i] = float4{0.f, 0.f, 0.f, 0.f};
      if (u < NU && tok < nt) {
        const size_t off = (size_t)(t0 + tok) * D + d4;
        if constexpr (sizeof(T) == 2) {
          const uint2 a = *reinterpret_cast<const uint2*>(kh + off);
          const uint2 b = *reinterpret_cast<const uint2*>(qh + off);
          rk[i] = float4{bf2f(a.x & 0xffffu), bf2f(a.x >> 16), bf2f(a.y & 0xffffu), bf2f(a.y >> 16)};
          rq[i] = float4{bf2f(b.x & 0xffffu), bf2f(b.x >> 16), bf2f(b.y & 0xffffu), bf2f(b.y >> 16)};
        } else {
          rk[i] = *reinterpret_cast<const float4*>(kh + off);
          rq[i] = *reinterpret_cast<const float4*>(qh + off);
        }
      }
    }
    {  // v: 64 tokens x 16 rows = 256 units of 4
      const int tok = tid >> 2, c4 = (tid & 3) * 4;
      rv = float4{0.f, 0.f, 0.f, 0.f};
      if (tok < nt) {
        const T* src = vh + (size_t)(t0 + tok) * M + 16 * rg + c4;
        rv = float4{ld_scalar<T>(src), ld_scalar<T>(src + 1), ld_scalar<T>(src + 2), ld_scalar<T>(src + 3)};
      }
    }
    rb = (tid < nt) ? ld_scalar<T>(bhp + t0 + tid) : 0.f;
  };

  prefetch(0, min(DTB, N));
  for (int t0 = 0; t0 < N; t0 += DTB) {
    const int nt = min(DTB, N - t0);
    // Stage: kh = phi(k)/sum phi(k), qh likewise (lanes of one token row are an
    // aligned group of UPT lanes).  Tokens past the end are staged as zero k, q
    // and beta, which leave W unchanged, so the sequential loop always runs 64.
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = tid + 256 * i;
      if (u < NU) {  // uniform per group of UPT lanes
        const int tok = u / UPT, d4 = (u % UPT) * 4;
        const bool ok = tok < nt;
        float4 a{phi(rk[i].x), phi(rk[i].y), phi(rk[i].z), phi(rk[i].w)};
        float4 b{phi(rq[i].x), phi(rq[i].y), phi(rq[i].z), phi(rq[i].w)};
        float sa = a.x + a.y + a.z + a.w, sb = b.x + b.y + b.z + b.w;
        if constexpr (UPT == 16) {
          sa = sum16(sa);
          sb = sum16(sb);
        } else {
          sa = sum8(sa);
          sb = sum8(sb);
        }
        const float ia = ok ? 1.f / sa : 0.f, ib = ok ? 1.f / sb : 0.f;
        *reinterpret_cast<float4*>(&Kh[tok][d4]) = float4{a.x * ia, a.y * ia, a.z * ia, a.w * ia};
        *reinterpret_cast<float4*>(&Qh[tok][d4]) = float4{b.x * ib, b.y * ib, b.z * ib, b.w * ib};
      }
    }
    {
      const int tok = tid >> 2, c4 = (tid & 3) * 4;
      *reinterpret_cast<float4*>(&Vs[tok][c4]) = rv;
    }
    if (tid < DTB) Bs[tid] = rb;
    __syncthreads();
    if (t0 + DTB < N) prefetch(t0 + DTB, min(DTB, N - t0 - DTB));

    // Sequential phase: one memory row per 16-lane group.  The chain from one
    // token to the next is v̄ = W k, the row's sum16, c = beta (v - v̄) and the
    // rank-1 write; the operands of token i + 1 are read from LDS while token
    // i runs, and o = W q hangs off the chain.  Lane n keeps the outputs of the
    // tokens i = n (mod 16) in registers until the block ends.
    const int row = 4 * w + rl;
    float kv[DPL], qv[DPL], vm, bt;
    auto read_tok = [&](int i) __attribute__((always_inline)) {
      if constexpr (DPL % 4 == 0) {
        const float4* kp = reinterpret_cast<const float4*>(&Kh[i][n * DPL]);
        const float4* qp = reinterpret_cast<const float4*>(&Qh[i][n * DPL]);
#pragma unroll
        for (int e4 = 0; e4 < DPL / 4; ++e4) {
          const float4 x = kp[e4], y = qp[e4];
          kv[4 * e4] = x.x; kv[4 * e4 + 1] = x.y; kv[4 * e4 + 2] = x.z; kv[4 * e4 + 3] = x.w;
          qv[4 * e4] = y.x; qv[4 * e4 + 1] = y.y; qv[4 * e4 + 2] = y.z; qv[4 * e4 + 3] = y.w;
        }
      } else {
        static_assert(DPL == 2, "rows hold 2 or a multiple of 4 elements per lane");
        const float2 x = *reinterpret_cast<const float2*>(&Kh[i][n * DPL]);
        const float2 y = *reinterpret_cast<const float2*>(&Qh[i][n * DPL]);
        kv[0] = x.x; kv[1] = x.y;
        qv[0] = y.x; qv[1] = y.y;
      }
      vm = Vs[i][row];
      bt = Bs[i];
    };
    float oreg[DTB / 16];
#pragma unroll
    for (int j = 0; j < DTB / 16; ++j) oreg[j] = 0.f;
    read_tok(0);
#pragma unroll
    for (int i = 0; i < DTB; ++i) {
      float k_[DPL], q_[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        k_[e] = kv[e];
        q_[e] = qv[e];
      }
      const float v_ = vm, b_ = bt;
      if (i + 1 < DTB) read_tok(i + 1);
      // retrieve: pairwise tree over the lane's elements, then the row sum
      float pp[DPL / 2];
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) pp[e] = W[2 * e] * k_[2 * e] + W[2 * e + 1] * k_[2 * e + 1];
#pragma unroll
      for (int h = DPL / 4; h >= 1; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) pp[e] += pp[e + h];
      const float vbar = sum16(pp[0]);
      const float c = b_ * (v_ - vbar);  // beta (v - vbar)
#pragma unroll
      for (int e = 0; e < DPL; ++e) W[e] += c * k_[e];  // write
      // read with the updated memory
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) pp[e] = W[2 * e] * q_[2 * e] + W[2 * e + 1] * q_[2 * e + 1];
#pragma unroll
      for (int h = DPL / 4; h >= 1; h >>= 1)
#pragma unroll
        for (int e = 0; e < h; ++e) pp[e] += pp[e + h];
      const float om = sum16(pp[0]);
      oreg[i / 16] = n == (i % 16) ? om : oreg[i / 16];
    }
#pragma unroll
    for (int j = 0; j < DTB / 16; ++j) Os[16 * j + n][row] = oreg[j];
    __syncthreads();
    {  // coalesced output of the block's 16 columns
      const int tok = tid >> 2, c4 = (tid & 3) * 4;
      if (tok < nt) {
        T* dst = oh + (size_t)(t0 + tok) * M + 16 * rg + c4;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = to_elem<T>(Os[tok][c4 + e]);
      }
    }
    // The next staging writes Kh/Qh/Vs/Bs only after every wave has passed the
    // barrier above, i.e. finished reading them; Os is rewritten only after the
    // next block's sequential phase, behind the next barrier.
    __syncthreads();
  }
  if (W_out) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) W_out[((size_t)bh * M + m) * D + n * DPL + e] = W[e];
  }
}

template <typename T, int D, int M>
static hipError_t deltanet_impl(const void* q, const void* k, const void* v, const void* beta, void* o, int BH,
                                int N, const float* W0, float* W_out, hipStream_t stream) {
  const unsigned nb = (unsigned)BH * (M / 16);
  hipLaunchKernelGGL((deltanet_kernel<T, D, M>), dim3(nb), dim3(256), 0, stream, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)beta, (T*)o, N, W0, W_out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Single-token step (the RNN form of the same rule), in place on W.  The step
// is a pure memory stream: every (b, h) reads and writes its M x D float32
// memory once (16 KiB each way at D = M = 64), so the kernel is bound by HBM
// bandwidth.  One wavefront owns one memory; lane l covers the four columns
// d = 4 (l % (D/4)) .. +3 of rows m = l / (D/4) + (256/D) p, so each load
// instruction of the wave reads 1 KiB of consecutive memory.  kh and qh are
// normalised with a reduction over the D/4 lanes of a row group; every row's
// retrieval and read are reductions over the same lanes.
template <typename T, int D, int M>
__global__ __launch_bounds__(256) void deltanet_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, const T* __restrict__ beta,
                                                            T* __restrict__ o, float* __restrict__ W, int BH) {
  constexpr int LPR = D / 4;     // lanes per memory row
  constexpr int RPP = 64 / LPR;  // rows per pass
  constexpr int NP = M / RPP;    // passes
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;  // whole wavefront; the kernel has no barrier
  const int dc = lane % LPR, r0 = lane / LPR;
  auto row_sum = [](float x) __attribute__((always_inline)) {
    if constexpr (LPR == 16) return sum16(x);
    else return sum8(x);
  };

  float* Wh = W + (size_t)bh * M * D + 4 * dc;
  float4 w[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) w[p] = *reinterpret_cast<const float4*>(Wh + (size_t)(r0 + RPP * p) * D);
  float vr[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) vr[p] = ld_scalar<T>(v + (size_t)bh * M + r0 + RPP * p);
  const float b = ld_scalar<T>(beta + bh);

  float4 kk = load4<T>(k + (size_t)bh * D + 4 * dc);
  float4 qq = load4<T>(q + (size_t)bh * D + 4 * dc);
  kk = float4{phi(kk.x), phi(kk.y), phi(kk.z), phi(kk.w)};
  qq = float4{phi(qq.x), phi(qq.y), phi(qq.z), phi(qq.w)};
  const float ik = 1.f / row_sum((kk.x + kk.y) + (kk.z + kk.w));
  const float iq = 1.f / row_sum((qq.x + qq.y) + (qq.z + qq.w));
  kk = float4{kk.x * ik, kk.y * ik, kk.z * ik, kk.w * ik};
  qq = float4{qq.x * iq, qq.y * iq, qq.z * iq, qq.w * iq};

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float vbar = row_sum((w[p].x * kk.x + w[p].y * kk.y) + (w[p].z * kk.z + w[p].w * kk.w));  // retrieve
    const float c = b * (vr[p] - vbar);                                                            // beta (v - vbar)
    w[p] = float4{w[p].x + c * kk.x, w[p].y + c * kk.y, w[p].z + c * kk.z, w[p].w + c * kk.w};     // write
    const float om = row_sum((w[p].x * qq.x + w[p].y * qq.y) + (w[p].z * qq.z + w[p].w * qq.w));  // read
    if (dc == 0) o[(size_t)bh * M + r0 + RPP * p] = to_elem<T>(om);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) *reinterpret_cast<float4*>(Wh + (size_t)(r0 + RPP * p) * D) = w[p];
}

template <typename T, int D, int M>
static hipError_t deltanet_step_impl(const void* q, const void* k, const void* v, const void* beta, void* o, float* W,
                                     int BH, hipStream_t stream) {
  const unsigned nb = (unsigned)((BH + 3) / 4);
  hipLaunchKernelGGL((deltanet_step_kernel<T, D, M>), dim3(nb), dim3(256), 0, stream, (const T*)q, (const T*)k,
                     (const T*)v, (const T*)beta, (T*)o, W, BH);
  return hipGetLastError();
}

hipError_t launch_deltanet_step(const void* q, const void* k, const void* v, const void* beta, void* o, float* W,
                                int BH, int D, int M, int bf16, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (bf16) {
    LA_DISPATCH_DM(deltanet_step_impl, bf16_t, q, k, v, beta, o, W, BH, stream)
  } else {
    LA_DISPATCH_DM(deltanet_step_impl, float, q, k, v, beta, o, W, BH, stream)
  }
}

// Copies W0 to W_out, or zero-fills it (empty sequence).
__global__ __launch_bounds__(256) void memory_copy_kernel(const float* W0, float* W_out, long long n) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < n) W_out[e] = W0 ? W0[e] : 0.f;
}

// Sequences run through the chunk-parallel kernels unless
// LINATTN_DELTANET_PATH=sequential selects the token-by-token kernel (one
// wavefront-reduction chain per row of W; it needs no workspace).  The variable
// is read at every call, by the workspace query and by the launch alike, so a
// call made with a workspace sized for the other path is still validated
// against the path it takes.
static bool deltanet_chunked() {
  const char* e = getenv("LINATTN_DELTANET_PATH");
  return !(e && strcmp(e, "sequential") == 0);
}

size_t deltanet_ws_bytes(int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0 || !deltanet_chunked()) return 0;
  return deltanet_chunk_ws_bytes(BH, N, D, M);
}

hipError_t launch_deltanet(const void* q, const void* k, const void* v, const void* beta, void* o, int BH, int N,
                           int D, int M, int bf16, const float* W0, float* W_out, void* ws, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (N == 0) {
    if (!W_out) return hipSuccess;
    const long long n = (long long)BH * M * D;
    hipLaunchKernelGGL(memory_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, W0, W_out, n);
    return hipGetLastError();
  }
  if (deltanet_chunked()) return launch_deltanet_chunked(q, k, v, beta, o, BH, N, D, M, bf16, W0, W_out, ws, stream);
  if (bf16) {
    LA_DISPATCH_DM(deltanet_impl, bf16_t, q, k, v, beta, o, BH, N, W0, W_out, stream)
  } else {
    LA_DISPATCH_DM(deltanet_impl, float, q, k, v, beta, o, BH, N, W0, W_out, stream)
  }
}

}  // namespace la
