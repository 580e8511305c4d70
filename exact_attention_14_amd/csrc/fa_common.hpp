// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

// log2(e): the kernels evaluate exp(x) as exp2(x * log2 e).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32x16 bf16 matrix-core step, D = A B + C.
// A (32 x 16): lane l holds row l%32, reduction slots 8*(l/32) .. +7.
// B (16 x 32): lane l holds column l%32, reduction slots 8*(l/32) .. +7.
// C/D (32 x 32): lane l holds column l%32; element v is row
//   8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32);
}

}  // namespace fa
