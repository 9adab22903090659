// Device-side helpers shared by the libdflash kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef _Float16 f16;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

#define DF_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16 x) { return static_cast<float>(x); }
// Round to nearest even (the gfx950 conversion instruction rounds this way).
__device__ __forceinline__ bf16 f2bf(float x) { return static_cast<bf16>(x); }

// Sum over the `width` lanes of an aligned lane group (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Reductions over the four lanes {l, l^16, l^32, l^48} using the gfx950
// permlane swaps (no LDS traffic). permlane32_swap(x, x) yields (lo|lo, hi|hi)
// and permlane16_swap(x, x) yields (row0|row0|row2|row2, row1|row1|row3|row3).
__device__ __forceinline__ float xrow4_max(float v) {
  int x = __float_as_int(v);
  auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  x = __float_as_int(v);
  auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float xrow4_sum(float v) {
  int x = __float_as_int(v);
  auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  v = __int_as_float(a[0]) + __int_as_float(a[1]);
  x = __float_as_int(v);
  auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dflash
