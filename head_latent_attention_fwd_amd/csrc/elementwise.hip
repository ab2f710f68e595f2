// Row-wise and element-wise kernels of the MLA path: RMSNorm + RoPE, the RoPE
// table, e4m3 quantisation (activations 1x128, weights 128x128), the top-k
// selection bitmask and the decode cache append.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

__device__ __forceinline__ float ld(const void* p, int dt, int64_t i) {
  return dt == DT_F32 ? ((const float*)p)[i] : bf2f(((const uint16_t*)p)[i]);
}
// input element i of a row-wise kernel: one array, or the sum of split-K partials
// (summed in split order; up to 16 partials are loaded before the first add)
__device__ __forceinline__ float ld_in(const NormRopeArgs& a, int64_t i) {
  if (a.in_splits <= 1) return ld(a.in, a.in_dtype, i);
  const float* p = (const float*)a.in;
  float v = p[i];
  if (a.in_splits <= 16) {
    float t[15];
#pragma unroll
    for (int s = 1; s < 16; ++s) t[s - 1] = s < a.in_splits ? p[(int64_t)s * a.split_stride + i] : 0.f;
#pragma unroll
    for (int s = 1; s < 16; ++s)
      if (s < a.in_splits) v += t[s - 1];
    return v;
  }
  for (int s = 1; s < a.in_splits; ++s) v += p[(int64_t)s * a.split_stride + i];
  return v;
}
__device__ __forceinline__ void st(void* p, int dt, int64_t i, float v) {
  if (dt == DT_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = f2bf(v);
}

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, red[i]);
  return t;
}

// RMSNorm (gamma * x / sqrt(mean(x^2) + eps)) over the row prefix and rotate-half
// RoPE on rope_heads 64-wide slices; one 256-thread block per row. Rows up to
// 256 * NORM_PT wide are read once into registers.
constexpr int NORM_PT = 8;
__global__ __launch_bounds__(256) void rmsnorm_rope_kernel(NormRopeArgs a, int rope_len) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int64_t ib = (int64_t)row * a.ld_in, ob = (int64_t)row * a.ld_out;
  if (a.norm_dim > 0 && a.norm_dim <= 256 * NORM_PT) {
    // the row stays in registers: one read of the input (and its partials)
    float v[NORM_PT];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NORM_PT; ++j) {
      const int i = tid + 256 * j;
      v[j] = i < a.norm_dim ? ld_in(a, ib + i) : 0.f;
      ss = fmaf(v[j], v[j], ss);
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)a.norm_dim + a.eps);
#pragma unroll
    for (int j = 0; j < NORM_PT; ++j) {
      const int i = tid + 256 * j;
      if (i < a.norm_dim) st(a.out, a.out_dtype, ob + i, a.gamma[i] * (v[j] * r));
    }
  } else if (a.norm_dim > 0) {
    float ss = 0.f;
    for (int i = tid; i < a.norm_dim; i += 256) {
      float v = ld_in(a, ib + i);
      ss = fmaf(v, v, ss);
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)a.norm_dim + a.eps);
    for (int i = tid; i < a.norm_dim; i += 256)
      st(a.out, a.out_dtype, ob + i, a.gamma[i] * (ld_in(a, ib + i) * r));
  }
  if (a.rope_heads > 0 && a.norm_dim == 0 && a.in_dtype == DT_BF16 && a.out_dtype == DT_BF16 && a.in_splits <= 1 &&
      !a.kpe && ((a.rope_off | a.rope_stride | a.ld_in | a.ld_out) & 3) == 0 &&
      (((uintptr_t)a.in | (uintptr_t)a.out | (uintptr_t)a.cos_tab | (uintptr_t)a.sin_tab) & 15) == 0) {
    // bf16 rotation only (the query's rope slices): 4 pairs per thread step,
    // 8-byte accesses
    const int pos = a.pos ? a.pos[row] : row % a.pos_period;
    const bool ok = pos >= 0 && pos < rope_len;
    for (int p = tid; p < a.rope_heads * 8; p += 256) {
      const int h = p >> 3, d0 = (p & 7) * 4;
      const int64_t o = a.rope_off + (int64_t)h * a.rope_stride + d0;
      const uint2 u1 = *(const uint2*)((const uint16_t*)a.in + ib + o);
      const uint2 u2 = *(const uint2*)((const uint16_t*)a.in + ib + o + 32);
      float4 c = make_float4(0.f, 0.f, 0.f, 0.f), sn = c;
      if (ok) {
        c = *(const float4*)&a.cos_tab[pos * 32 + d0];
        sn = *(const float4*)&a.sin_tab[pos * 32 + d0];
      }
      const float x1[4] = {__uint_as_float(u1.x << 16), __uint_as_float(u1.x & 0xffff0000u),
                           __uint_as_float(u1.y << 16), __uint_as_float(u1.y & 0xffff0000u)};
      const float x2[4] = {__uint_as_float(u2.x << 16), __uint_as_float(u2.x & 0xffff0000u),
                           __uint_as_float(u2.y << 16), __uint_as_float(u2.y & 0xffff0000u)};
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y1[e] = x1[e] * cc[e] - x2[e] * ss[e];
        y2[e] = x2[e] * cc[e] + x1[e] * ss[e];
      }
      *(uint2*)((uint16_t*)a.out + ob + o) = make_uint2(pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]));
      *(uint2*)((uint16_t*)a.out + ob + o + 32) = make_uint2(pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]));
    }
  } else if (a.rope_heads > 0) {
    const int pos = a.pos ? a.pos[row] : row % a.pos_period;
    const bool ok = pos >= 0 && pos < rope_len;
    for (int p = tid; p < a.rope_heads * 32; p += 256) {
      const int h = p >> 5, d = p & 31;
      const int64_t o = a.rope_off + (int64_t)h * a.rope_stride + d;
      const float x1 = ld_in(a, ib + o), x2 = ld_in(a, ib + o + 32);
      float c = 0.f, s = 0.f;
      if (ok) { c = a.cos_tab[pos * 32 + d]; s = a.sin_tab[pos * 32 + d]; }
      const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
      st(a.out, a.out_dtype, ob + o, y1);
      st(a.out, a.out_dtype, ob + o + 32, y2);
      if (a.kpe) {
        const int bb = row / a.pos_period, t = row - bb * a.pos_period;
        const int64_t kb = ((int64_t)bb * a.kpe_tp + t) * 64 + d;
        st(a.kpe, a.out_dtype, kb, y1);
        st(a.kpe, a.out_dtype, kb + 32, y2);
      }
    }
  }
}

// The two RMSNorms of a down-projection row and the RoPE of its k_pe; one
// 256-thread block per row, 4 consecutive elements per thread-chunk (16-byte
// fp32 / 8-byte bf16 accesses), both sums of squares in one block reduction.
constexpr int QKV_CH = 4;   // chunks of 4 per thread: rows up to 4096 wide
__global__ __launch_bounds__(256) void qkv_norm_kernel(QkvNormArgs a) {
  __shared__ float red[2][4];
  __shared__ float kpe_s[64];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nq = a.Dq >> 2, nkv = a.L >> 2, nch = nq + nkv + 16;
  float4 v[QKV_CH];
  float sq = 0.f, skv = 0.f;
#pragma unroll
  for (int j = 0; j < QKV_CH; ++j) {
    const int c = tid + 256 * j;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < (a.kpe_in ? nq + nkv : nch)) {   // (k_pe from its own partials below)
      const int64_t i = (int64_t)row * a.ld_in + 4 * c;
      if (a.in_dtype == DT_F32) {
        const float* p = (const float*)a.in + i;
        float4 t[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s < a.in_splits) t[s] = *(const float4*)(p + (int64_t)s * a.split_stride);
        x = t[0];
#pragma unroll
        for (int s = 1; s < 8; ++s)
          if (s < a.in_splits) { x.x += t[s].x; x.y += t[s].y; x.z += t[s].z; x.w += t[s].w; }
        for (int s = 8; s < a.in_splits; ++s) {
          const float4 u = *(const float4*)(p + (int64_t)s * a.split_stride);
          x.x += u.x; x.y += u.y; x.z += u.z; x.w += u.w;
        }
      } else {
        const uint2 u = *(const uint2*)((const uint16_t*)a.in + i);
        x = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                        __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
      }
      const float q2 = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      if (c < nq) sq += q2;
      else if (c < nq + nkv) skv += q2;
      else *(float4*)&kpe_s[4 * (c - nq - nkv)] = x;
    }
    v[j] = x;
  }
  if (a.kpe_in && tid < 16) {   // k_pe: the sum of its split-K partials, in split order
    const float* p = a.kpe_in + (int64_t)row * 64 + 4 * tid;
    float4 x = *(const float4*)p;
    for (int s = 1; s < a.kpe_splits; ++s) {
      const float4 u = *(const float4*)(p + (int64_t)s * a.kpe_split_stride);
      x.x += u.x; x.y += u.y; x.z += u.z; x.w += u.w;
    }
    *(float4*)&kpe_s[4 * tid] = x;
  }
  sq = wave_sum(sq);
  skv = wave_sum(skv);
  if (lane == 0) { red[0][wave] = sq; red[1][wave] = skv; }
  __syncthreads();
  sq = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  skv = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float rq = 1.0f / sqrtf(sq / (float)a.Dq + a.eps), rkv = 1.0f / sqrtf(skv / (float)a.L + a.eps);
  int P, bb = 0;
  if (a.pos) {
    P = a.pos[row];
  } else {
    bb = row / a.pos_period;
    P = a.pos_off + row - bb * a.pos_period;
  }
  uint16_t* kv = nullptr;
  if (a.kv_pos_stride > 0) {
    if (P >= 0 && P < a.kv_pos_max) kv = (uint16_t*)a.kv_out + (int64_t)row * a.ld_kv + (int64_t)P * a.kv_pos_stride;
  } else if (a.kv_batch_stride > 0) {
    kv = (uint16_t*)a.kv_out + (int64_t)bb * a.kv_batch_stride + (int64_t)P * a.ld_kv;
  } else {
    kv = (uint16_t*)a.kv_out + (int64_t)row * a.ld_kv;
  }
  uint16_t* q = (uint16_t*)a.q_out + (int64_t)row * a.ld_q;
#pragma unroll
  for (int j = 0; j < QKV_CH; ++j) {
    const int c = tid + 256 * j;
    if (c < nq) {
      const float4 g = *(const float4*)&a.gq[4 * c];
      const uint2 pk = make_uint2(pack_bf16x2(g.x * (v[j].x * rq), g.y * (v[j].y * rq)),
                                  pack_bf16x2(g.z * (v[j].z * rq), g.w * (v[j].w * rq)));
      *(uint2*)(q + 4 * c) = pk;
      if (a.q_codes) {   // 32 consecutive lanes hold one 128-wide group
        const float y0 = __uint_as_float(pk.x << 16), y1 = __uint_as_float(pk.x & 0xffff0000u);
        const float y2 = __uint_as_float(pk.y << 16), y3 = __uint_as_float(pk.y & 0xffff0000u);
        float amax = fmaxf(fmaxf(fabsf(y0), fabsf(y1)), fmaxf(fabsf(y2), fabsf(y3)));
        amax = xor16_max(row16_max(amax));
        e4m3_quotients(amax, true, [&](const float s, auto quo) {
          uint32_t code = 0u;
          if (s != 0.f)
            code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                quo(y2), quo(y3), __builtin_amdgcn_cvt_pk_fp8_f32(quo(y0), quo(y1), 0, false), true);
          *(uint32_t*)(a.q_codes + (int64_t)row * a.Dq + 4 * c) = code;
          if ((c & 31) == 0) a.q_scales[(int64_t)row * (a.Dq >> 7) + (c >> 5)] = s;
        });
      }
    } else if (c < nq + nkv && kv) {
      const int e = 4 * (c - nq);
      const float4 g = *(const float4*)&a.gkv[e];
      uint2 pk = make_uint2(pack_bf16x2(g.x * (v[j].x * rkv), g.y * (v[j].y * rkv)),
                            pack_bf16x2(g.z * (v[j].z * rkv), g.w * (v[j].w * rkv)));
      if (a.kv_codes || a.kv_view) {   // as for q: 32 consecutive lanes hold one 128-wide group
        const float y0 = __uint_as_float(pk.x << 16), y1 = __uint_as_float(pk.x & 0xffff0000u);
        const float y2 = __uint_as_float(pk.y << 16), y3 = __uint_as_float(pk.y & 0xffff0000u);
        float amax = fmaxf(fmaxf(fabsf(y0), fabsf(y1)), fmaxf(fabsf(y2), fabsf(y3)));
        amax = xor16_max(row16_max(amax));
        e4m3_quotients(amax, true, [&](const float s, auto quo) {
          uint32_t code = 0u;
          if (s != 0.f)
            code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                quo(y2), quo(y3), __builtin_amdgcn_cvt_pk_fp8_f32(quo(y0), quo(y1), 0, false), true);
          if (a.kv_codes) {
            *(uint32_t*)(a.kv_codes + (int64_t)row * a.L + e) = code;
            if (((c - nq) & 31) == 0) a.kv_scales[(int64_t)row * (a.L >> 7) + ((c - nq) >> 5)] = s;
          }
          if (a.kv_view) {   // the entry holds the value kv_b's quantiser maps the latent to
            const float2v d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false);
            const float2v d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, true);
            pk = make_uint2(pack_bf16x2(d0[0] * s, d0[1] * s), pack_bf16x2(d1[0] * s, d1[1] * s));
          }
        });
      }
      *(uint2*)(kv + e) = pk;
    }
  }
  if (tid < 32) {
    const int d = tid;
    const bool ok = P >= 0 && P < a.rope_len;
    const float c = ok ? a.cos_tab[P * 32 + d] : 0.f, sn = ok ? a.sin_tab[P * 32 + d] : 0.f;
    const float x1 = kpe_s[d], x2 = kpe_s[d + 32];
    const float y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
    if (kv) {
      kv[a.L + d] = f2bf(y1);
      kv[a.L + d + 32] = f2bf(y2);
    }
    if (a.kpe) {
      uint16_t* kp = (uint16_t*)a.kpe + ((int64_t)bb * a.kpe_tp + P) * 64;
      kp[d] = f2bf(y1);
      kp[d + 32] = f2bf(y2);
    }
  }
}

// Batched transpose through a 64 x 65 LDS tile.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* src, int64_t sld, int64_t sb, uint16_t* dst,
                                                          int64_t dld, int64_t db, int rows, int cols) {
  __shared__ uint16_t t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, z = blockIdx.z;
  const uint16_t* S = src + z * sb;
  uint16_t* D = dst + z * db;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if (r0 + r < rows && c0 + c < cols) t[r][c] = S[(int64_t)(r0 + r) * sld + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;
    if (r0 + r < rows && c0 + c < cols) D[(int64_t)(c0 + c) * dld + r0 + r] = t[r][c];
  }
}

// SwiGLU product of a stacked gate | up row and its e4m3 codes: 8 columns per
// thread, 16 threads per 128-wide group (max over the group by shuffles).
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(const void* gu, int64_t ld, int nsplit,
                                                             int64_t split_stride, int rows, int cols, uint8_t* hq,
                                                             float* hs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = cols / 8;
  if (i >= (int64_t)rows * cpr) return;   // whole 16-lane groups leave together (cols % 128 == 0)
  const int64_t r = i / cpr;
  const int c = (int)(i - r * cpr) * 8;
  float gf[8], uf[8];
  if (nsplit > 0) {   // fp32 partials, summed in split order (gate and up products rounded to bf16)
    const float* p = (const float*)gu + r * ld + c;
#pragma unroll
    for (int e = 0; e < 8; ++e) { gf[e] = 0.f; uf[e] = 0.f; }
    for (int sp = 0; sp < nsplit; ++sp) {
      const float4 g0 = *(const float4*)(p + sp * split_stride), g1 = *(const float4*)(p + sp * split_stride + 4);
      const float4 u0 = *(const float4*)(p + sp * split_stride + cols);
      const float4 u1 = *(const float4*)(p + sp * split_stride + cols + 4);
      gf[0] += g0.x; gf[1] += g0.y; gf[2] += g0.z; gf[3] += g0.w; gf[4] += g1.x; gf[5] += g1.y; gf[6] += g1.z;
      gf[7] += g1.w;
      uf[0] += u0.x; uf[1] += u0.y; uf[2] += u0.z; uf[3] += u0.w; uf[4] += u1.x; uf[5] += u1.y; uf[6] += u1.z;
      uf[7] += u1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { gf[e] = bf2f(f2bf(gf[e])); uf[e] = bf2f(f2bf(uf[e])); }
  } else {
    const uint16_t* b = (const uint16_t*)gu + r * ld + c;
    const uint4 gv = *(const uint4*)b, uv = *(const uint4*)(b + cols);
    const uint16_t* ge = (const uint16_t*)&gv;
    const uint16_t* ue = (const uint16_t*)&uv;
#pragma unroll
    for (int e = 0; e < 8; ++e) { gf[e] = bf2f(ge[e]); uf[e] = bf2f(ue[e]); }
  }
  float y[8], amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y[e] = bf2f(f2bf(gf[e] / (1.0f + __builtin_amdgcn_exp2f(-gf[e] * 1.4426950408889634f)) * uf[e]));
    amax = fmaxf(amax, fabsf(y[e]));
  }
  amax = row16_max(amax);
  e4m3_quotients(amax, true, [&](const float sc, auto quo) {
    uint2 code = make_uint2(0u, 0u);
    if (sc != 0.f) {
      code.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(y[2]), quo(y[3]),
                                                          __builtin_amdgcn_cvt_pk_fp8_f32(quo(y[0]), quo(y[1]), 0, false),
                                                          true);
      code.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(y[6]), quo(y[7]),
                                                          __builtin_amdgcn_cvt_pk_fp8_f32(quo(y[4]), quo(y[5]), 0, false),
                                                          true);
    }
    *(uint2*)(hq + r * cols + c) = code;
    if ((c & 127) == 0) hs[r * (cols / 128) + c / 128] = sc;
  });
}

// Strided row copy, one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint16_t* src, int64_t sld, uint16_t* dst, int64_t dld,
                                                        int64_t rows, int cpr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cpr) return;
  const int64_t r = i / cpr;
  const int c = (int)(i - r * cpr);
  *(uint4*)(dst + r * dld + 8 * c) = *(const uint4*)(src + r * sld + 8 * c);
}

// h = silu(g) * u, 8 bf16 values per thread (the unfused SwiGLU path).
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint4* g, const uint4* u, uint4* h, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 gv = g[i], uv = u[i];
  const uint16_t* ge = (const uint16_t*)&gv;
  const uint16_t* ue = (const uint16_t*)&uv;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gf = bf2f(ge[e]);
    y[e] = gf / (1.0f + __builtin_amdgcn_exp2f(-gf * 1.4426950408889634f)) * bf2f(ue[e]);
  }
  h[i] = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
}

// kpe[b, t, :] = cache[b, t, kpe_off : kpe_off + 64] for t < P, one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void gather_kpe_kernel(const uint16_t* cache, int64_t cache_ld, int row_ld,
                                                         int kpe_off, int B, int P, uint16_t* kpe, int Tp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * P * 8) return;
  const int c = (int)(i & 7);
  const int64_t bt = i >> 3;
  const int b = (int)(bt / P), t = (int)(bt - (int64_t)b * P);
  *(uint4*)(kpe + ((int64_t)b * Tp + t) * 64 + 8 * c) =
      *(const uint4*)(cache + (int64_t)b * cache_ld + (int64_t)t * row_ld + kpe_off + 8 * c);
}

// Zero the padding keys t in [T, Tp) of kn [B,H,Tp,128], vt [B,H,128,Tp], kpe [B,Tp,64].
template <typename E>
__global__ __launch_bounds__(256) void zero_kv_padding_kernel(E* kn, E* vt, E* kpe, int H, int T, int Tp) {
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H, pad = Tp - T;
  E* k = kn + ((int64_t)bh * Tp + T) * 128;
  for (int i = threadIdx.x; i < pad * 128; i += 256) k[i] = E(0);
  E* v = vt + (int64_t)bh * 128 * Tp;
  for (int i = threadIdx.x; i < pad * 128; i += 256) v[(int64_t)(i / pad) * Tp + T + i % pad] = E(0);
  if (h == 0) {
    E* p = kpe + ((int64_t)b * Tp + T) * 64;
    for (int i = threadIdx.x; i < pad * 64; i += 256) p[i] = E(0);
  }
}

__global__ void rope_table_kernel(float* c, float* s, int n_pos, double base) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pos * 32) return;
  const int p = i >> 5, d = i & 31;
  const double th = (double)p * pow(base, -(double)d / 32.0);
  c[i] = (float)cos(th);
  s[i] = (float)sin(th);
}

__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// 16 lanes per (row, 128-group), 8 consecutive values per lane: s = amax/448,
// q = e4m3(x / s) (fp32 quotient, round to nearest even, saturating). A
// 256-thread block covers 16 consecutive (row, group) pairs in row-major order.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* a, int64_t lda, int dt, int M, int K,
                                                          uint8_t* q, float* scales) {
  const int G = K / 128, tid = threadIdx.x, sub = tid & 15;
  const int64_t pair = (int64_t)blockIdx.x * 16 + (tid >> 4);
  if (pair >= (int64_t)M * G) return;   // whole 16-lane groups leave together
  const int m = (int)(pair / G), g = (int)(pair - (int64_t)m * G);
  const int64_t base = (int64_t)m * lda + g * 128 + sub * 8;
  float v[8];
  if (dt == DT_F32) {
    const float4 x0 = *(const float4*)((const float*)a + base), x1 = *(const float4*)((const float*)a + base + 4);
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w; v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  } else {
    const uint4 u = *(const uint4*)((const uint16_t*)a + base);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = row16_max(amax);   // within the 16 lanes
  e4m3_quotients(amax, dt != DT_F32, [&](const float s, auto quo) {
    uint2 code = make_uint2(0u, 0u);
    if (s != 0.f) {
      code.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(v[2]), quo(v[3]),
                                                          __builtin_amdgcn_cvt_pk_fp8_f32(quo(v[0]), quo(v[1]), 0, false),
                                                          true);
      code.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quo(v[6]), quo(v[7]),
                                                          __builtin_amdgcn_cvt_pk_fp8_f32(quo(v[4]), quo(v[5]), 0, false),
                                                          true);
    }
    *(uint2*)(q + (int64_t)m * K + g * 128 + sub * 8) = code;
    if (sub == 0) scales[(int64_t)m * G + g] = s;
  });
}

// One block per 128x128 weight block.
__global__ __launch_bounds__(256) void quant_block128_kernel(const float* w, int N, int K, uint8_t* q,
                                                             float* scales) {
  __shared__ float red[4];
  const int nb = blockIdx.y, kb = blockIdx.x, tid = threadIdx.x;
  const int n0 = nb * 128, k0 = kb * 128;
  float amax = 0.f;
  for (int e = tid; e < 128 * 128; e += 256) {
    const int n = n0 + (e >> 7), k = k0 + (e & 127);
    if (n < N && k < K) amax = fmaxf(amax, fabsf(w[(int64_t)n * K + k]));
  }
  amax = block_max(amax, red);
  const float s = amax / 448.0f;
  for (int e = tid * 2; e < 128 * 128; e += 512) {
    const int n = n0 + (e >> 7), k = k0 + (e & 127);
    if (n >= N || k >= K) continue;
    const float v0 = w[(int64_t)n * K + k];
    const float v1 = (k + 1 < K) ? w[(int64_t)n * K + k + 1] : 0.f;
    const uint32_t code = s != 0.f ? to_e4m3x2(v0 / s, v1 / s) : 0u;
    q[(int64_t)n * K + k] = (uint8_t)(code & 0xFF);
    if (k + 1 < K) q[(int64_t)n * K + k + 1] = (uint8_t)(code >> 8);
  }
  if (tid == 0) scales[(int64_t)nb * ((K + 127) / 128) + kb] = s;
}

// One block per query row: OR the picks (t <= s) into LDS words, then store.
__global__ __launch_bounds__(256) void topk_bitmask_kernel(const int32_t* idx, int T, int k, int P, int Tk,
                                                            uint32_t* mask) {
  extern __shared__ uint32_t words[];
  const int s = blockIdx.x, b = blockIdx.y, W = (Tk + 31) / 32;
  for (int i = threadIdx.x; i < W; i += 256) words[i] = 0u;
  __syncthreads();
  const int32_t* row = idx + ((int64_t)b * T + s) * k;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int t = row[j];
    if (t >= 0 && t <= P + s && t < Tk) atomicOr(&words[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  uint32_t* out = mask + ((int64_t)b * T + s) * W;
  for (int i = threadIdx.x; i < W; i += 256) out[i] = words[i];
}

}  // namespace

hipError_t launch_rmsnorm_rope(const NormRopeArgs& a, hipStream_t s) {
  // Positions outside the table (only possible through a device pos array)
  // give zero rotations instead of reading past it.
  if (a.rows <= 0) return hipSuccess;
  rmsnorm_rope_kernel<<<a.rows, 256, 0, s>>>(a, a.rope_len);
  return hipGetLastError();
}

// Each 128-wide latent group of a cache row replaced, in place, by the value its
// dynamic 1x128 e4m3 quantisation stands for (bf16 of code x scale): the input
// kv_b's quantiser sees, and a fixed point of that quantiser. 16 lanes per
// group, 8 values (16 bytes) per lane; the group maximum of |x| on the bf16 bit
// patterns (for finite values their order is that of |x|).
__global__ __launch_bounds__(256) void latent_view_kernel(uint16_t* __restrict__ cache, int64_t groups, int gpr,
                                                          int64_t stride) {
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (gid >= groups) return;   // whole 16-lane rows leave together
  const int64_t row = gid / gpr;
  uint4* p = (uint4*)(cache + row * stride + (gid - row * gpr) * 128) + (threadIdx.x & 15);
  const uint4 v = *p;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t am = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t m = w[e] & 0x7fff7fffu;
    am = max(am, max(m & 0xffffu, m >> 16));
  }
  const float amax = row16_max(__uint_as_float(am << 16));
  e4m3_quotients(amax, true, [&](const float s, auto quo) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      int code = 0;
      if (s != 0.f)
        code = __builtin_amdgcn_cvt_pk_fp8_f32(
            quo(__uint_as_float(w[e + 1] << 16)), quo(__uint_as_float(w[e + 1] & 0xffff0000u)),
            __builtin_amdgcn_cvt_pk_fp8_f32(quo(__uint_as_float(w[e] << 16)), quo(__uint_as_float(w[e] & 0xffff0000u)),
                                            0, false),
            true);
      const float2v d0 = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
      const float2v d1 = __builtin_amdgcn_cvt_pk_f32_fp8(code, true);
      o[e] = pack_bf16x2(d0[0] * s, d0[1] * s);
      o[e + 1] = pack_bf16x2(d1[0] * s, d1[1] * s);
    }
    *p = make_uint4(o[0], o[1], o[2], o[3]);
  });
}

hipError_t launch_qkv_norm(const QkvNormArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if ((a.Dq & 3) || (a.L & 3) || (a.ld_in & 3) || (a.Dq + a.L + 64) / 4 > 256 * QKV_CH ||
      (a.in_dtype != DT_F32 && a.in_dtype != DT_BF16) || (a.in_dtype == DT_F32 && (a.split_stride & 3)) ||
      (a.ld_q & 3) || (a.ld_kv & 3) || (a.kv_pos_stride & 3) || a.in_splits < 1 || (!a.pos && a.pos_period <= 0) ||
      (a.q_codes && ((a.Dq & 127) || !a.q_scales || ((uintptr_t)a.q_codes & 3))) ||
      (a.kv_codes && ((a.Dq & 127) || (a.L & 127) || !a.kv_scales || ((uintptr_t)a.kv_codes & 3))) ||
      (a.kpe_in && (a.kpe_splits < 1 || a.kpe_splits > 8 || ((uintptr_t)a.kpe_in & 15) || (a.kpe_split_stride & 3))) ||
      (a.kv_view && ((a.Dq & 127) || (a.L & 127))))
    return hipErrorInvalidValue;
  qkv_norm_kernel<<<a.rows, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_latent_e4m3_view(void* cache, int64_t rows, int64_t stride, int L, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((L & 127) || L <= 0 || stride < L || (stride & 7) || ((uintptr_t)cache & 15)) return hipErrorInvalidValue;
  const int64_t groups = rows * (L / 128);
  latent_view_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>((uint16_t*)cache, groups, L / 128, stride);
  return hipGetLastError();
}

hipError_t launch_zero_kv_padding(void* kn, void* vt, void* kpe, int B, int H, int T, int Tp, int elem_bytes,
                                  hipStream_t s) {
  if (Tp == T) return hipSuccess;
  if (elem_bytes == 4)
    zero_kv_padding_kernel<float><<<B * H, 256, 0, s>>>((float*)kn, (float*)vt, (float*)kpe, H, T, Tp);
  else
    zero_kv_padding_kernel<uint16_t><<<B * H, 256, 0, s>>>((uint16_t*)kn, (uint16_t*)vt, (uint16_t*)kpe, H, T, Tp);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* c, float* sn, int n_pos, float base, hipStream_t s) {
  if (n_pos <= 0) return hipSuccess;
  rope_table_kernel<<<(n_pos * 32 + 255) / 256, 256, 0, s>>>(c, sn, n_pos, (double)base);
  return hipGetLastError();
}

hipError_t launch_quant_1x128(const void* a, int64_t lda, int a_dtype, int M, int K, uint8_t* q, float* scales,
                              hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((lda & 7) || (((uintptr_t)a | (uintptr_t)q) & 15)) return hipErrorInvalidValue;   // 16-byte row pieces
  const int64_t pairs = (int64_t)M * (K / 128);
  quant_1x128_kernel<<<(unsigned)((pairs + 15) / 16), 256, 0, s>>>(a, lda, a_dtype, M, K, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_block128(const float* w, int N, int K, uint8_t* q, float* scales, hipStream_t s) {
  dim3 grid((K + 127) / 128, (N + 127) / 128);
  quant_block128_kernel<<<grid, 256, 0, s>>>(w, N, K, q, scales);
  return hipGetLastError();
}

hipError_t launch_transpose16(const uint16_t* src, int64_t sld, int64_t sb, uint16_t* dst, int64_t dld, int64_t db,
                              int rows, int cols, int batch, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  transpose16_kernel<<<grid, 256, 0, s>>>(src, sld, sb, dst, dld, db, rows, cols);
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const void* gu, int64_t ld, int nsplit, int64_t split_stride, int rows, int cols,
                                 uint8_t* hq, float* hs, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((cols & 127) || (ld & 7) || ld < 2 * cols || (split_stride & 3) || nsplit < 0 ||
      (((uintptr_t)gu | (uintptr_t)hq) & 15))
    return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (cols / 8);
  silu_mul_quant_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(gu, ld, nsplit, split_stride, rows, cols, hq,
                                                                    hs);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const uint16_t* src, int64_t sld, uint16_t* dst, int64_t dld, int64_t rows, int cols,
                            hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if ((cols & 7) || (sld & 7) || (dld & 7) || (((uintptr_t)src | (uintptr_t)dst) & 15)) return hipErrorInvalidValue;
  const int64_t n = rows * (cols / 8);
  copy_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, sld, dst, dld, rows, cols / 8);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* g, const void* u, void* h, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n8 = n / 8;
  silu_mul_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>((const uint4*)g, (const uint4*)u, (uint4*)h, n8);
  return hipGetLastError();
}

hipError_t launch_topk_bitmask(const int32_t* idx, int B, int T, int k, int P, int Tk, uint32_t* mask, hipStream_t s) {
  if (P < 0 || Tk < P + T || (Tk + 31) / 32 * 4 > 65536) return hipErrorInvalidValue;
  dim3 grid(T, B);
  topk_bitmask_kernel<<<grid, 256, ((Tk + 31) / 32) * 4, s>>>(idx, T, k, P, Tk, mask);
  return hipGetLastError();
}

hipError_t launch_gather_kpe(const void* cache, int64_t cache_ld, int row_ld, int kpe_off, int B, int P, void* kpe,
                             int Tp, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  if (P > Tp || (row_ld & 7) || (kpe_off & 7) || (cache_ld & 7) || (((uintptr_t)cache | (uintptr_t)kpe) & 15))
    return hipErrorInvalidValue;
  const int64_t n = (int64_t)B * P * 8;   // 16-byte chunks
  gather_kpe_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint16_t*)cache, cache_ld, row_ld, kpe_off, B,
                                                                P, (uint16_t*)kpe, Tp);
  return hipGetLastError();
}

}  // namespace mla
