// Row-major bf16 tiles in LDS for the gfx950 MFMA kernels: a 16-byte-unit XOR
// swizzle, 16- and 8-byte unit access, and transposed fragment reads with
// ds_read_b64_tr_b16.
//
// Operand layouts (lane l = 16 g + n of a 64-lane wavefront, MFMA 16x16x32 bf16):
//  * d-contraction: lane group g holds d = 32 s + 8 g + e (e < 8) of slab s, read
//    as one 16-byte unit of a row-major tile row.
//  * j-contraction: lane group g holds j = 32 s + 16 h + 4 g + r (e = 4 h + r),
//    the rows an accumulator tile keeps in the lane, read from a row-major tile
//    with ds_read_b64_tr_b16 (within a 16-lane group the instruction returns
//    out[i][e] = in[4 e + i / 4][i % 4]).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace la {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Row term of the swizzle: with row = 8d + 4a + 2b + c (low bits), the unit
// index of a 16-byte unit is XORed with
//   U = 8: (b, a^c, a^d) as bits (2, 1, 0);   U = 4: (a^b, a^d) as bits (1, 0).
// It depends on the row only modulo 16.  Under either LDS bank width (32 or 64
// four-byte banks per cycle) it leaves these patterns free of bank conflicts:
//  * 16-byte unit reads of one unit in 16 consecutive rows (MFMA operands),
//  * 16-byte unit stores of whole consecutive rows,
//  * ds_read_b64_tr_b16 over 16 consecutive rows and two adjacent units.
// (The earlier row ^ row >> 3 term serialised the transposed reads two-way on a
// 32-bank LDS; measured by the SQ_LDS_BANK_CONFLICT counter.)
template <int U>
__host__ __device__ constexpr int row_swz(int row) {
  static_assert(U == 4 || U == 8, "tiles have 4 or 8 units per row");
  const int a = (row >> 2) & 1, b = (row >> 1) & 1, c = row & 1, d = (row >> 3) & 1;
  return U == 8 ? (b << 2) | ((a ^ c) << 1) | (a ^ d) : ((a ^ b) << 1) | (a ^ d);
}

// Swizzled element offset of (row, col) in a row-major bf16 tile with U 16-byte
// units per row: unit (col / 8) is XORed with row_swz(row).
template <int U>
__host__ __device__ __forceinline__ int swz(int row, int col) {
  const int unit = (col >> 3) ^ row_swz<U>(row);
  return row * U * 8 + unit * 8 + (col & 7);
}

// The swizzle splits into a per-lane part and a part fixed at compile time.  For
// element (R + r, C + c) with R a multiple of 16, C a multiple of 8, and (C >> 3)
// and (c >> 3) sharing no bit (so their sum carries nothing):
//   2 * swz<U>(R + r, C + c) == (lane_off<U>(r, c) ^ xor_off<U>(C)) + 16 U R.
// The lane part is formed once per kernel; every access is then one XOR (none
// when the XOR term is 0) and an immediate offset.
template <int U>
__host__ __device__ constexpr uint32_t lane_off(int r, int c) {
  return (uint32_t)(16 * U * r + 2 * (c & 7) + 16 * (((c >> 3) ^ row_swz<U>(r)) & (U - 1)));
}
template <int U>
__host__ __device__ constexpr uint32_t xor_off(int C) {
  return (uint32_t)(16 * ((C >> 3) & (U - 1)));
}
// Address of (R + r, C + c) from the lane part of (r, c).
template <int U, typename T>
__device__ __forceinline__ T* tile_at(T* tile, uint32_t lane, int R, int C) {
  typedef typename std::conditional<std::is_const<T>::value, const char, char>::type byte;
  return reinterpret_cast<T*>(reinterpret_cast<byte*>(tile) + 16 * U * R + (lane ^ xor_off<U>(C)));
}

// j-slot fragment as jfrag below, from the lane part ltr = lane_off<U>(4 g + n / 4, 4 (n % 4))
// and a column base col0 (a multiple of 16): rows rbase + 32-row slab (rbase a multiple of 16).
template <int U>
__device__ __forceinline__ bf16x8 jfrag_at(const bf16_t* tile, uint32_t ltr, int rbase, int col0) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tile_at<U>(tile, ltr, rbase, col0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tile_at<U>(tile, ltr, rbase + 16, col0));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return as_bf16x8(u32x4{x[0], x[1], y[0], y[1]});
}

// 16-byte unit (row, col..col+7) of a swizzled tile; col is a multiple of 8.
template <int U>
__device__ __forceinline__ u32x4& unit16(bf16_t* tile, int row, int col) {
  return reinterpret_cast<u32x4*>(tile)[swz<U>(row, col) >> 3];
}
template <int U>
__device__ __forceinline__ const u32x4& unit16(const bf16_t* tile, int row, int col) {
  return reinterpret_cast<const u32x4*>(tile)[swz<U>(row, col) >> 3];
}
// 8-byte half unit (row, col..col+3); col is a multiple of 4.
template <int U>
__device__ __forceinline__ u32x2& unit8(bf16_t* tile, int row, int col) {
  return reinterpret_cast<u32x2*>(tile)[swz<U>(row, col) >> 2];
}

// Two floats -> two bf16 (round to nearest even) in one dword, lo first.
__device__ __forceinline__ uint32_t cvt_pk(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}

__device__ __forceinline__ float lo_of(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_of(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transposed fragment: lane (n, g) gets rows row0 + 4g + e (e < 4) of column col0 + n
// from a row-major swizzled tile.
template <int U>
__device__ __forceinline__ u32x2 tr_read(const bf16_t* tile, int row0, int col0, int g, int sl) {
  const int row = row0 + 4 * g + (sl >> 2);
  const int col = col0 + 4 * (sl & 3);
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + swz<U>(row, col)));
  return __builtin_bit_cast(u32x2, r);
}

// j-slot fragment (8 rows 32s + 16h + 4g + r of column col0 + n) from a row-major tile.
template <int U>
__device__ __forceinline__ bf16x8 jfrag(const bf16_t* tile, int rbase, int col0, int g, int sl) {
  const u32x2 a = tr_read<U>(tile, rbase, col0, g, sl);
  const u32x2 b = tr_read<U>(tile, rbase + 16, col0, g, sl);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

__device__ __forceinline__ bf16x8 ones8() {
  const uint32_t one2 = 0x3F803F80u;
  return as_bf16x8(u32x4{one2, one2, one2, one2});
}

// phi of eight bf16 values (one 16-byte unit) split into a bf16 head and tail,
// phi = head + tail to about 2^-17 relative; invalid rows give zeros.
__device__ __forceinline__ void phi_split8(const u32x4& raw, bool ok, u32x4& hv, u32x4& lv) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t wd = raw[h];
    const float a = ok ? phi(lo_of(wd)) : 0.f, b = ok ? phi(hi_of(wd)) : 0.f;
    const uint32_t hp = cvt_pk(a, b);
    hv[h] = hp;
    lv[h] = cvt_pk(a - lo_of(hp), b - hi_of(hp));
  }
}

}  // namespace la
