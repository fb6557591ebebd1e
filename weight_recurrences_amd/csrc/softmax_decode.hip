// Softmax attention decode step over a key/value cache on gfx950: the
// comparison baseline for the recurrent form.
//
// "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器": Appendix C.1 compares linear attention's RNN form with a
// "stateful" softmax attention that keeps the keys and values of the earlier
// tokens instead of recomputing them; the attention itself is §3.1 eq.(2),
// softmax(q K^T / sqrt(D)) V.  One step appends the new token's key and value
// at row L of the cache and attends over rows 0..L.
//
// Unlike the linear decode step (a fixed D x M state per head), this step reads
// every cached token: (L + 1) (D + M) elements per head, so its cost grows with
// the context.  It is bound by HBM bandwidth.
//
// One workgroup of 256 threads (4 waves) per (batch, head).  A group of 8 lanes
// owns one key at a time (32 keys per round over the workgroup) and lane r of
// the group holds elements r D/8 .. and r M/8 .. of q, k and v; the score is an
// 8-lane DPP sum.  Each group keeps an online-softmax state (running maximum of
// the scores, in log2 units, their exponential sum, and its slice of the
// weighted value sum) and folds U rounds of keys per rescale.  The 32 partial
// states of a workgroup are merged through LDS.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace smx {

constexpr int NT = 256;  // threads per workgroup
constexpr int KPR = 32;  // keys per round (4 waves x 8 groups of 8 lanes)
constexpr int U = 2;     // rounds folded per rescale (rows in flight per lane): 2 keeps 76 VGPRs, 6 waves per SIMD

// E consecutive elements (16 or 8 bytes of bf16, 32 or 16 bytes of float32) as floats.
template <int E>
__device__ __forceinline__ void load_row(const bf16_t* p, float (&x)[E]) {
  static_assert(E == 4 || E == 8, "4 or 8 elements per lane");
  if constexpr (E == 8) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf2f(w[i] & 0xffffu);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      x[2 * i] = bf2f(w[i] & 0xffffu);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}
template <int E>
__device__ __forceinline__ void load_row(const float* p, float (&x)[E]) {
  static_assert(E == 4 || E == 8, "4 or 8 elements per lane");
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = w[e];
  }
}
// Copies E elements (one lane's slice of a row) unchanged.
template <typename T, int E>
__device__ __forceinline__ void copy_row(const T* src, T* dst) {
  constexpr int BYTES = E * (int)sizeof(T);
  if constexpr (BYTES == 32) {
    reinterpret_cast<u32x4*>(dst)[0] = reinterpret_cast<const u32x4*>(src)[0];
    reinterpret_cast<u32x4*>(dst)[1] = reinterpret_cast<const u32x4*>(src)[1];
  } else if constexpr (BYTES == 16) {
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  } else {
    *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(src);
  }
}

template <int M>
struct Smem {
  float m[KPR], l[KPR];
  float acc[KPR][M];
};

template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void softmax_decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, T* __restrict__ o,
                                                            T* __restrict__ Kc, T* __restrict__ Vc, int L, int Lmax) {
  constexpr int EK = D / 8, EV = M / 8;  // elements per lane of a key / value row
  __shared__ Smem<M> sm;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, grp = lane >> 3, r = lane & 7;
  const int slot = 8 * w + grp;  // this group's partial state
  const T* qh = q + (size_t)bh * D;
  const T* kh = k + (size_t)bh * D;
  const T* vh = v + (size_t)bh * M;
  T* Kh = Kc + (size_t)bh * Lmax * D;
  T* Vh = Vc + (size_t)bh * Lmax * M;

  // Append the new token at row L (the scores below take it from k and v).
  if (w == 0 && grp == 0) {
    copy_row<T, EK>(kh + r * EK, Kh + (size_t)L * D + r * EK);
    copy_row<T, EV>(vh + r * EV, Vh + (size_t)L * M + r * EV);
  }

  // q scaled by log2(e) / sqrt(D): scores come out in log2 units for exp2.
  float qs[EK];
  load_row<EK>(qh + r * EK, qs);
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
  for (int e = 0; e < EK; ++e) qs[e] *= qscale;

  float mx = -INFINITY, sum = 0.f, acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;

  for (int j0 = 0; j0 <= L; j0 += U * KPR) {
    if (j0 + slot > L) break;  // this group has no key left (uniform within the group)
    float kr[U][EK], vr[U][EV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * KPR + slot;
      if (j < L) {
        load_row<EK>(Kh + (size_t)j * D + r * EK, kr[u]);
        load_row<EV>(Vh + (size_t)j * M + r * EV, vr[u]);
      } else if (j == L) {
        load_row<EK>(kh + r * EK, kr[u]);
        load_row<EV>(vh + r * EV, vr[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EK; ++e) kr[u][e] = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) vr[u][e] = 0.f;
      }
    }
    float s[U];
    float bm = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) p += qs[e] * kr[u][e];
      p = sum8(p);
      s[u] = (j0 + u * KPR + slot <= L) ? p : -INFINITY;
      bm = fmaxf(bm, s[u]);
    }
    // One rescale per U rounds: bm is finite (the group's first key is valid).
    const float a = exp2f(mx - bm);
    sum *= a;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2f(s[u] - bm);
      sum += p;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] += p * vr[u][e];
    }
    mx = bm;
  }

  // Merge the 32 partial states: o = sum_i 2^(m_i - m) acc_i / sum_i 2^(m_i - m) l_i.
#pragma unroll
  for (int e = 0; e < EV; ++e) sm.acc[slot][r * EV + e] = acc[e];
  if (r == 0) {
    sm.m[slot] = mx;
    sm.l[slot] = sum;
  }
  __syncthreads();
  if (tid < M) {
    float gm = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < KPR; ++i) gm = fmaxf(gm, sm.m[i]);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int i = 0; i < KPR; ++i) {
      const float f = sm.l[i] == 0.f ? 0.f : exp2f(sm.m[i] - gm);  // groups without keys hold no weight
      num += f * sm.acc[i][tid];
      den += f * sm.l[i];
    }
    o[(size_t)bh * M + tid] = to_elem<T>(num / den);
  }
}

template <typename T, int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, void* o, void* Kc, void* Vc, int BH, int L,
                       int Lmax, hipStream_t stream) {
  hipLaunchKernelGGL((softmax_decode_kernel<T, D, M>), dim3((unsigned)BH), dim3(NT), 0, stream, (const T*)q,
                     (const T*)k, (const T*)v, (T*)o, (T*)Kc, (T*)Vc, L, Lmax);
  return hipGetLastError();
}

}  // namespace smx

hipError_t launch_softmax_decode(const void* q, const void* k, const void* v, void* o, void* Kc, void* Vc, int BH,
                                 int L, int Lmax, int D, int M, int bf16, hipStream_t stream) {
  if (BH == 0) return hipSuccess;
  if (bf16) {
    LA_DISPATCH_DM(smx::impl, bf16_t, q, k, v, o, Kc, Vc, BH, L, Lmax, stream)
  } else {
    LA_DISPATCH_DM(smx::impl, float, q, k, v, o, Kc, Vc, BH, L, Lmax, stream)
  }
}

}  // namespace la
