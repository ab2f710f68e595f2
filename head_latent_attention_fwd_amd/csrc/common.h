// Shared device helpers for the gfx950 kernels: storage types, bf16/fp32
// conversions, MFMA operand vector types and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));

// bf16 is carried as uint16_t in memory.
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (v_cvt_pk_bf16_f32)
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((float2v){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// word 3 of a gfx9 raw-buffer descriptor (32-bit data format, no swizzle, no stride)
constexpr int BUF_DW3 = 0x00020000;

// 32x32x16 bf16 MFMA: D[i][j] += sum_k A[i][k] B[k][j]. Lane l supplies row
// (l % 32) of A and column (l % 32) of B, each with 8 k values; the k values
// a lane supplies are the same set for A and B, so any consistent assignment
// of logical k to (lane / 32, slot) gives the full sum. Result: lane l holds
// column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA: lane l supplies row/column (l % 16) with 8 k values;
// result: lane l holds column (l % 16), rows 4*(l/16) + r for r = 0..3.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x64 e4m3 x e4m3 MFMA (32 bytes of k per lane, same lane rules).
__device__ __forceinline__ floatx16 mfma32_fp8(intx8 a, intx8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int row32(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
