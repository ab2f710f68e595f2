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

// Cross-lane reductions on the VALU: DPP moves within each row of 16 lanes
// (quad permutes lane ^ 1, lane ^ 2, then row rotations by 4 and 8), and the
// permlane swaps across rows (lane ^ 16, lane ^ 32). Every lane of the reduced
// set ends with the result; a reduced set must be wholly active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x124>(x);
  return x + dpp_mov<0x128>(x);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x124>(x));
  return fmaxf(x, dpp_mov<0x128>(x));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float wave_max(float v) { return xor32_max(xor16_max(row16_max(v))); }
__device__ __forceinline__ float wave_sum(float v) { return xor32_sum(xor16_sum(row16_sum(v))); }

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

// Quotients x / s of the e4m3 activation quantisers, s = amax / 448, for a
// group whose values x (|x| <= amax) and amax are bf16 values. For
// amax >= 2^-60 the correctly rounded reciprocal rc = 1 / s, q0 = x rc and one
// residual step q0 + (x - q0 s) rc (the residual exact in one FMA) equal the
// correctly rounded quotient for every such pair (checked exhaustively over
// all bf16 x and amax; quotients below 2^-12, code 0 either way, aside).
// Smaller groups, and values that are not bf16 (bf16_values = false), divide;
// an all-zero group (s = 0) gives zero quotients. body(s, quo) runs once with
// the quotient function the group takes, so the choice is one branch per group.
template <class Body>
__device__ __forceinline__ void e4m3_quotients(float amax, bool bf16_values, Body&& body) {
  const float s = amax / 448.0f;
  if (bf16_values && amax >= 0x1p-60f) {
    const float rc = 1.0f / s;
    body(s, [s, rc](float x) {
      const float q0 = x * rc;
      return __builtin_fmaf(__builtin_fmaf(-q0, s, x), rc, q0);
    });
  } else {
    body(s, [s](float x) { return s != 0.f ? x / s : 0.f; });
  }
}

// Stores marked non-temporal, for the large GEMM outputs (kv_b's k_nope /
// v^T, q_b's q, wo's output): written once, read by a later kernel, too big to
// stay in the caches anyway. Measured on the e4m3 prefill GEMMs: 3-10 % faster
// than plain stores.
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store((intx4){(int)v.x, (int)v.y, (int)v.z, (int)v.w}, (intx4*)p);
}

__device__ __forceinline__ int row32(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
