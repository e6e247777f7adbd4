// Device helpers shared by the libkvarn kernels (gfx950, wave64).
//
// Lane-level building blocks: MFMA operand types, DPP row rotations, the
// gfx950 permlane16/32 swaps (verified on hardware: permlane32_swap(a, b)
// leaves a = [a.lo32 | b.lo32], b = [a.hi32 | b.hi32]; permlane16_swap(a, b)
// leaves a = [a.r0, b.r0, a.r2, b.r2], b = [a.r1, b.r1, a.r3, b.r3] in rows of
// 16 lanes), and the record layout constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTok = 128;    // tokens per tile = page size
constexpr int kCh = 128;     // head_dim

// ---- record layout (see include/libkvarn.h) --------------------------------
__host__ __device__ constexpr int k_code_bytes(int kb) { return kTok * kCh * kb / 8; }
__host__ __device__ constexpr int v_code_bytes(int vb) { return kTok * kCh * vb / 8; }
__host__ __device__ constexpr int scale_offset(int kb, int vb) { return k_code_bytes(kb) + v_code_bytes(vb); }
// One half's scale block (floats): c[128], s'[ng][128], m'[ng][128]; ng = 128 / group.
__host__ __device__ constexpr int half_scale_floats(int ng) { return kCh * (1 + 2 * ng); }
__host__ __device__ constexpr int record_bytes(int kb, int vb, int ng) {
  return scale_offset(kb, vb) + 2 * half_scale_floats(ng) * 4;
}

// ---- lane primitives --------------------------------------------------------
__device__ __forceinline__ float as_f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u(float x) { return __builtin_bit_cast(uint32_t, x); }

// Value of lane (i - N) mod 16 within each row of 16 lanes (DPP row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, false));
}

// Sum / min / max over the 16 lanes of a row; every lane gets the same bits
// (each step combines x_i with x_{i-N}; the partial sums are periodic, so the
// operands only swap places between lanes).
__device__ __forceinline__ float row_sum16(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}
__device__ __forceinline__ float row_min16(float x) {
  x = fminf(x, row_ror<8>(x));
  x = fminf(x, row_ror<4>(x));
  x = fminf(x, row_ror<2>(x));
  x = fminf(x, row_ror<1>(x));
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<1>(x));
  return x;
}

__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}

// Reduce two values over lane bit 5: lanes 0-31 return sum_over_bit5(x),
// lanes 32-63 return sum_over_bit5(y).
__device__ __forceinline__ float red32(float x, float y) {
  swap32(x, y);
  return x + y;
}
// Reduce two values over lane bit 4: rows 0,2 return sum_over_bit4(x), rows 1,3 of y.
__device__ __forceinline__ float red16(float x, float y) {
  swap16(x, y);
  return x + y;
}
// Max over the 4 rows (lane bits 4 and 5); every lane gets the same value.
__device__ __forceinline__ float rows_max4(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum4(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap32(a, b);
  return a + b;
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// x with its mantissa cut to fp16's 10 bits (rounded toward zero), exact in fp32.  For
// 2^-14 <= |x| <= 65504 it is an fp16 value, so converting it to fp16 is exact whichever conversion
// instruction the compiler picks: an fp16 operand and the fp32 value its remainder or rounding error
// is computed from can then never disagree (two conversion instructions may break rounding ties
// differently).
__device__ __forceinline__ float f16_trunc(float x) { return as_f(as_u(x) & 0xFFFFE000u); }

}  // namespace kvarn
