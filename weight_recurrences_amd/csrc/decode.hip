// RNN-form single-token decode step on gfx950.
//
// "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.4 eq.(18)-(20): s <- s + phi(k) v^T, z <- z + phi(k),
// o = phi(q)^T s / phi(q)^T z, the state updated before it is read.
//
// The step is a pure state stream: every (b, h) reads and writes its D x M
// float32 matrix once (16 KiB each way at D = M = 64), so the kernel is bound
// by HBM bandwidth.  One wavefront owns one (b, h) state; lane l covers the
// four columns 4*(l % (M/4)) .. +3 of rows d = l / (M/4) + (256/M) * p, so each
// load instruction of the wave reads 1 KiB of consecutive memory.  The
// numerator is reduced across the lanes that share columns with cross-lane
// shuffles; the denominator is a full-wave sum of phi(q)_d z_d.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

template <typename T, int D, int M>
__global__ __launch_bounds__(256) void decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, T* __restrict__ o,
                                                          float* __restrict__ S, float* __restrict__ z, int BH) {
  constexpr int LPR = M / 4;     // lanes per state row
  constexpr int RPP = 64 / LPR;  // rows per pass
  constexpr int NP = D / RPP;    // passes
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;  // whole wavefront; the kernel has no barrier
  const int mc = lane % LPR, r0 = lane / LPR;

  // The state's loads go out first, then the token's and z's (with the token's
  // loads first, the compiler waits for k and q to apply phi while half of the
  // state's loads are not yet issued: +1.1 us per step from cold caches).
  float* Sh = S + (size_t)bh * D * M + 4 * mc;
  float4 s[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) s[p] = *reinterpret_cast<const float4*>(Sh + (size_t)(r0 + RPP * p) * M);
  const int dl = lane < D ? lane : 0;  // lanes past D re-read element 0 (unused)
  const float kraw = ld_scalar<T>(k + (size_t)bh * D + dl);
  const float qraw = ld_scalar<T>(q + (size_t)bh * D + dl);
  const float zraw = z[(size_t)bh * D + dl];
  const float4 vv = load4<T>(v + (size_t)bh * M + 4 * mc);
  const float pk = lane < D ? phi(kraw) : 0.f;
  const float pq = lane < D ? phi(qraw) : 0.f;

  float4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int d = r0 + RPP * p;
    const float kd = __shfl(pk, d);
    const float qd = __shfl(pq, d);
    s[p].x += kd * vv.x;
    s[p].y += kd * vv.y;
    s[p].z += kd * vv.z;
    s[p].w += kd * vv.w;
    acc.x += qd * s[p].x;
    acc.y += qd * s[p].y;
    acc.z += qd * s[p].z;
    acc.w += qd * s[p].w;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) *reinterpret_cast<float4*>(Sh + (size_t)(r0 + RPP * p) * M) = s[p];

#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }

  float zd = 0.f;
  if (lane < D) {
    zd = zraw + pk;
    z[(size_t)bh * D + lane] = zd;
  }
  const float den = wave_sum(pq * zd);
  if (r0 == 0) {
    const float inv = 1.f / den;
    store4<T>(o + (size_t)bh * M + 4 * mc, float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv});
  }
}

template <typename T, int D, int M>
static hipError_t decode_impl(const void* q, const void* k, const void* v, void* o, float* S, float* z, int BH,
                              hipStream_t stream) {
  const unsigned nb = (unsigned)((BH + 3) / 4);
  hipLaunchKernelGGL((decode_step_kernel<T, D, M>), dim3(nb), dim3(256), 0, stream, (const T*)q, (const T*)k,
                     (const T*)v, (T*)o, S, z, BH);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* S, float* z, int BH, int D,
                         int M, int bf16, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (bf16) {
    LA_DISPATCH_DM(decode_impl, bf16_t, q, k, v, o, S, z, BH, stream)
  } else {
    LA_DISPATCH_DM(decode_impl, float, q, k, v, o, S, z, BH, stream)
  }
}

}  // namespace la
