// Device helpers shared by the gfx950 kernels: bf16 conversion, the feature
// map, MFMA wrappers and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef uint16_t bf16_t;  // bfloat16 stored as its raw bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
// Branch-free: both results are formed and selected.
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? nan : r;
}

// Two floats -> two bf16 packed in one dword (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

// phi(x) = elu(x) + 1 with alpha = 1 ("Transformers are RNNs", §3.2.1 eq.(7)):
// x + 1 for x > 0, exp(x) otherwise (the exp form keeps relative accuracy for
// very negative x).  Evaluated branch-free as max(min(exp(x), 1), x + 1): since
// exp(x) >= 1 + x with equality only at 0, this is x + 1 for x > 0 and exp(x)
// for x <= 0 (up to one rounding of exp near 0, where the two agree within an
// ulp); -inf maps to 0 and NaN propagates.  The min is the clamp modifier of
// v_exp_f32 and the max one v_maximum3_f32 (IEEE maximum, NaN-propagating): five
// VALU instructions with the unpack, and no compare and select.
__device__ __forceinline__ float phi(float x) {
  const float e = __builtin_amdgcn_fmed3f(__expf(x), 0.f, 1.f);
  return __builtin_elementwise_maximum(e, x + 1.f);
}

template <typename T> __device__ __forceinline__ float ld_scalar(const T* p);
template <> __device__ __forceinline__ float ld_scalar<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_scalar<bf16_t>(const bf16_t* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ T to_elem(float f);
template <> __device__ __forceinline__ float to_elem<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t to_elem<bf16_t>(float f) { return (bf16_t)f2bf(f); }

// Four consecutive elements as float4 (bf16 widened exactly) and back (bf16
// rounded to nearest even).
template <typename T> __device__ __forceinline__ float4 load4(const T* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return float4{bf2f(w.x & 0xffffu), bf2f(w.x >> 16), bf2f(w.y & 0xffffu), bf2f(w.y >> 16)};
}
template <typename T> __device__ __forceinline__ void store4(T* p, float4 x);
template <> __device__ __forceinline__ void store4<float>(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 x) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf2(x.x, x.y), pack_bf2(x.z, x.w)};
}


// ---- MFMA (16x16 output tiles, 64 lanes: lane = 16*g + n) --------------------
// A operand: lane (n, g) holds row n, k-slots of group g.  B operand: lane
// (n, g) holds column n, the same k-slots.  Result: lane (n, g) holds rows
// 4g..4g+3 of column n (element r of the f32x4).
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- cross-lane reductions ---------------------------------------------------
// DPP controls (GFX9 encoding).
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <- lane 15-i within 16

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets it.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  x += dpp<DPP_MIRROR>(x);
  return x;
}

// Sum over each aligned group of 8 lanes.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  return x;
}

// Sum over the whole wavefront (all 64 lanes get it).
__device__ __forceinline__ float wave_sum(float x) {
  x = sum16(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
