// Query absorption of the latent-space decode step (DeepSeek-V3.2-Exp · Sparse
// attention, "Explanation": the key up-projection is folded into the query so
// a decoded token scores cached latents directly):
//   q_lat[b, h, 0:512]   = q_nope[b, h, :] . W_UK_h      (W_UK_h = Wkv_b rows [256h, 256h+128), [128, 512])
//   q_lat[b, h, 512:576] = RoPE(q_pe[b, h, :], cache_len[b])
//
// One 512-thread workgroup per (head, half of the 512 latent columns, 128
// sequences). Its half of W_UK_h, [128 j, 256 c] (64 KB), moves HBM -> LDS
// with 16-byte direct-to-LDS loads, two 512-byte rows per load instruction,
// 16-byte chunks XOR-permuted within aligned groups of 16 by
// ((j & 3) << 2) | ((j >> 2) & 3). The product C^T[c, b] = W_UK_h^T[c, j] .
// q^T[j, b] runs on v_mfma_f32_32x32x16_bf16 with W_UK_h^T read by
// ds_read_b64_tr_b16 and q read straight from global memory, one 16-byte load
// per K step (the k slots of half hi of step ks are rows 16 ks + 8 hi + 0..7).
// Wave w covers c in [256 z + 128 (w & 1), +128) and sequences [32 (w >> 1),
// +32) of the tile. The results go back through LDS (the W half's space, as
// [128 sequences][256 c] bf16, 16-byte chunk k of row r at k ^ (r & 31)) so
// that each sequence's 512-byte piece of q_lat is written by 32 adjacent
// 16-byte stores. The q_pe rotation of the tile is split between the two
// halves by pair index.
//
// With e4m3 weights the half tile is read as codes, expanded to bf16 (exact:
// every e4m3 value is a bf16 value) and written to LDS in the same layout; the
// contraction runs over W_UK_h's 128 rows, which lie in one 128x128 scale block
// row, so the block scale of each 128-column group multiplies the result.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swj(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }
__device__ __forceinline__ v4s read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}

template <bool FP8>
__global__ __launch_bounds__(512, 2) void decode_absorb_kernel(const uint16_t* __restrict__ q,
                                                               const void* __restrict__ wkv_b,
                                                               const float* __restrict__ w_scale,
                                                               uint16_t* __restrict__ qlat,
                                                               const int32_t* __restrict__ cache_len,
                                                               const float* __restrict__ cos_tab,
                                                               const float* __restrict__ sin_tab, int B, int H,
                                                               int max_len) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[128 * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, z = blockIdx.y, b0 = blockIdx.z * 128;

  if constexpr (FP8) {
    // codes -> bf16 -> LDS: thread handles 16-byte pieces (row j, 16 columns 16 qc..) of the half
    const uint8_t* W8 = (const uint8_t*)wkv_b + (int64_t)h * 256 * 512 + 256 * z;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 512 * i, j = idx >> 4, qc = idx & 15;
      v[i] = *(const uint4*)(W8 + (int64_t)j * 512 + qc * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 512 * i, j = idx >> 4, qc = idx & 15;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], false);
        const float2v up = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], true);
        o[2 * e] = pack_bf16x2(lo[0], lo[1]);
        o[2 * e + 1] = pack_bf16x2(up[0], up[1]);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ch = 2 * qc + half;
        *(uint4*)(sw + j * 256 + ((((ch & 15) ^ swj(j)) | (ch & 16)) << 3)) =
            make_uint4(o[4 * half], o[4 * half + 1], o[4 * half + 2], o[4 * half + 3]);
      }
    }
  } else {
    // W_UK_h half -> LDS: load i of wave w fills rows j = 16 i + 2 w + (lane >> 5)
    const uint16_t* W = (const uint16_t*)wkv_b + (int64_t)h * 256 * 512 + 256 * z;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 16 * i + 2 * wave + (lane >> 5);
      __builtin_amdgcn_global_load_lds(W + (int64_t)j * 512 + (((lane & 31) ^ swj(j)) << 3),
                                       sw + (16 * i + 2 * wave) * 256, 16, 0, 0);
    }
  }

  // q fragments (B operand): lane (sequence l32, half hi) holds, for k-step
  // ks, q_nope dims 16 ks + 8 hi + 0..7
  const int l32 = lane & 31, hi = lane >> 5, wc = wave & 1, wb = wave >> 1;
  const int bq = b0 + wb * 32 + l32;
  bf16x8 qf[8];
  {
    const uint16_t* qp = q + ((int64_t)min(bq, B - 1) * H + h) * 192 + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qp + 16 * ks);
  }

  // q_pe rotation: thread handles pair d = 16 z + (tid & 15) of sequences
  // b0 + (tid >> 4) + 32 u; every load is issued before the first store
  {
    const int d = 16 * z + (tid & 15);
    int P[4];
    float x1[4], x2[4], c[4], sn[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = min(b0 + (tid >> 4) + 32 * u, B - 1);
      P[u] = cache_len[b];
      const uint16_t* src = q + ((int64_t)b * H + h) * 192 + 128;
      x1[u] = bf2f(src[d]);
      x2[u] = bf2f(src[d + 32]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = P[u] >= 0 && P[u] < max_len;
      c[u] = ok ? cos_tab[P[u] * 32 + d] : 0.f;
      sn[u] = ok ? sin_tab[P[u] * 32 + d] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + (tid >> 4) + 32 * u;
      if (b < B) {
        uint16_t* o = qlat + ((int64_t)b * H + h) * 576 + 512;
        o[d] = f2bf(x1[u] * c[u] - x2[u] * sn[u]);
        o[d + 32] = f2bf(x2[u] * c[u] + x1[u] * sn[u]);
      }
    }
  }
  __syncthreads();

  // W^T fragments: 16-lane group g reads rows j = 16 ks + 8 (g >> 1) + 4 e + (lane % 16) / 4,
  // columns c = 128 wc + 32 cb + 16 (g & 1) + 4 (lane % 4) of the half
  const int g = lane >> 4, L = lane & 15;
  floatx16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int c = 128 * wc + 32 * cb + 16 * (g & 1) + 4 * (L & 3);
      const int j0 = 16 * ks + 8 * (g >> 1) + (L >> 2), j1 = j0 + 4;
      const int ch = c >> 3;   // 16-byte chunk of column c
      const uint16_t* p0 = sw + j0 * 256 + ((((ch & 15) ^ swj(j0)) | (ch & 16)) << 3) + (c & 7);
      const uint16_t* p1 = sw + j1 * 256 + ((((ch & 15) ^ swj(j1)) | (ch & 16)) << 3) + (c & 7);
      const v4s lo = read_tr(p0), up = read_tr(p1);
      const bf16x8 wf = __builtin_bit_cast(bf16x8, (v8s){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
      acc[cb] = mfma32(wf, qf[ks], acc[cb]);
    }
  // lane: sequence bq, dims c = 256 z + 128 wc + 32 cb + 8 rg + 4 hi + 0..3
  if constexpr (FP8) {   // block (2h, 2z + wc) of the [2H, 4] scale grid
    const float sc = w_scale[(int64_t)2 * h * 4 + 2 * z + wc];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] *= sc;
  }
  __syncthreads();   // every wave is done reading the W half
  {
    const int r = wb * 32 + l32;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int k = 16 * wc + 4 * cb + rg;   // 16-byte chunk of c = 128 wc + 32 cb + 8 rg
        *(uint2*)(sw + r * 256 + ((k ^ (r & 31)) << 3) + 4 * hi) =
            make_uint2(pack_bf16x2(acc[cb][4 * rg], acc[cb][4 * rg + 1]),
                       pack_bf16x2(acc[cb][4 * rg + 2], acc[cb][4 * rg + 3]));
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // pass i: rows 16 i + tid / 32, chunk tid % 32
    const int r = 16 * i + (tid >> 5), k = tid & 31;
    if (b0 + r < B)
      *(uint4*)(qlat + ((int64_t)(b0 + r) * H + h) * 576 + 256 * z + 8 * k) =
          *(const uint4*)(sw + r * 256 + ((k ^ (r & 31)) << 3));
  }
}

}  // namespace

hipError_t launch_decode_absorb(const void* q, const void* wkv_b, const float* w_scale, void* qlat,
                                const int32_t* cache_len, const float* cos_tab, const float* sin_tab, int B, int H,
                                int max_len, hipStream_t s) {
  dim3 grid(H, 2, (B + 127) / 128);
  if (w_scale)
    decode_absorb_kernel<true><<<grid, 512, 0, s>>>((const uint16_t*)q, wkv_b, w_scale, (uint16_t*)qlat, cache_len,
                                                    cos_tab, sin_tab, B, H, max_len);
  else
    decode_absorb_kernel<false><<<grid, 512, 0, s>>>((const uint16_t*)q, wkv_b, nullptr, (uint16_t*)qlat,
                                                     cache_len, cos_tab, sin_tab, B, H, max_len);
  return hipGetLastError();
}

}  // namespace mla

// ---------------------------------------------------------------------------
// Value un-absorption of the latent-space decode step:
//   o[b, 128 h + j] = sum_c W_UV_h[j, c] o_lat[b, h, c]    (W_UV_h = Wkv_b rows [256h + 128, 256h + 256))
// with o_lat merged here from the attention's per-split partials:
//   o_lat = sum_s w_s part_s / sum_s w_s,  w_s = exp2(lse_s - max_s lse_s)   (split order)
// (splits == 1: o_lat is read as is). With e4m3 weights the product is the
// block-scaled one of the dequantised weight: W_UV_h's codes are expanded
// exactly to bf16 and the block scale of column group g = c / 128 is folded
// into o_lat's group g before it is rounded to bf16 for the MFMA.
//
// One 256-thread workgroup per (head h, block of 64 rows b); wave w takes
// rows 16w..16w+15 and all 128 j on v_mfma_f32_16x16x32_bf16 (W_UV_h as the
// first operand, so a lane's results are 4 consecutive j of one row). W_UV_h
// [128 j, 512 c] sits in LDS as bf16 (128 KB), 16-byte chunk ch of row j at
// chunk ch ^ (j & 15) of the row. Outputs: o in bf16 (staged through LDS so
// that each row's 256-byte piece goes out as 16 adjacent 16-byte stores) and,
// for an e4m3 wo, o's codes and its scale per (row, head) (one 1x128 group),
// quantised from the bf16 values.
namespace mla {
namespace {

__global__ __launch_bounds__(256, 1) void decode_unabsorb_kernel(UnabsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[128 * 512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b0 = blockIdx.y * 64;
  const int H = a.H;
  const bool fp8 = a.w_scale != nullptr;
  // this lane's row for the B operand: b = b0 + 16 wave + lane % 16, k chunk lane / 16
  const int g4 = lane >> 4, L = lane & 15;
  const int bq = b0 + 16 * wave + L;
  const bool row_ok = bq < a.B;
  const int64_t rh = (int64_t)min(bq, a.B - 1) * H + h;
  const int64_t rows = (int64_t)a.B * H;
  const uint16_t* part = (const uint16_t*)a.part;
  // One run: the lane's 16 o_lat fragments are loaded before W_UV_h is staged
  // so that both are in flight together.
  uint4 frag[16];
  if (a.splits == 1) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) frag[ks] = *(const uint4*)(part + rh * 512 + 32 * ks + 8 * g4);
  }
  if (fp8) {   // codes -> bf16 -> LDS: 16-byte piece i of the thread = row j, codes 16 cc .. 16 cc + 15
    const uint8_t* W8 = (const uint8_t*)a.wkv_b + ((int64_t)256 * h + 128) * 512;
    uint4 wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, cc = idx & 31;
      wv[i] = *(const uint4*)(W8 + (int64_t)j * 512 + 16 * cc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = tid + 256 * i, j = idx >> 5, cc = idx & 31;
      const uint32_t w[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
      uint32_t o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], false);
        const float2v up = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[e], true);
        o[2 * e] = pack_bf16x2(lo[0], lo[1]);
        o[2 * e + 1] = pack_bf16x2(up[0], up[1]);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ch = 2 * cc + half;
        *(uint4*)(sw + j * 512 + ((ch ^ (j & 15)) << 3)) =
            make_uint4(o[4 * half], o[4 * half + 1], o[4 * half + 2], o[4 * half + 3]);
      }
    }
  } else {   // bf16 rows straight to LDS: load i of wave w fills row j = 4 i + w (one 1 KB row)
    const uint16_t* W = (const uint16_t*)a.wkv_b + ((int64_t)256 * h + 128) * 512;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) {
      const int j = 4 * i + wave, ch = lane;   // lane fills physical chunk `lane`
      __builtin_amdgcn_global_load_lds(W + (int64_t)j * 512 + ((ch ^ (j & 15)) << 3), sw + j * 512, 16, 0, 0);
    }
  }
  // run weights exp2(lse_s - max) are recomputed where used (no indexed register array)
  float mx = -INFINITY, den = 0.f;
  if (a.splits > 1) {
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.lse[s * rows + rh]);
    if (mx != -INFINITY)
      for (int s = 0; s < a.splits; ++s) den += __builtin_amdgcn_exp2f(a.lse[s * rows + rh] - mx);
  }
  const float inv = a.splits > 1 ? (den > 0.f ? 1.f / den : 0.f) : 1.f;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // W_UV_h landed in LDS (direct loads)
  __syncthreads();

  floatx4 acc[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[jt][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int c0 = 32 * ks + 8 * g4;   // the 8 columns of this lane's k slots
    bf16x8 bfr;
    if (a.splits == 1 && !fp8) {
      bfr = __builtin_bit_cast(bf16x8, frag[ks]);
    } else {
      float f[8];
      if (a.splits == 1) {
        const uint32_t p[4] = {frag[ks].x, frag[ks].y, frag[ks].z, frag[ks].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(p[e] << 16);
          f[2 * e + 1] = __uint_as_float(p[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
        if (mx != -INFINITY)
          for (int s = 0; s < a.splits; ++s) {
            const float ws = __builtin_amdgcn_exp2f(a.lse[s * rows + rh] - mx);
            const uint4 u = *(const uint4*)(part + (s * rows + rh) * 512 + c0);
            const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              f[2 * e] += ws * __uint_as_float(p[e] << 16);
              f[2 * e + 1] += ws * __uint_as_float(p[e] & 0xffff0000u);
            }
          }
      }
      float sc = inv;
      if (fp8) sc *= a.w_scale[(int64_t)(2 * h + 1) * 4 + (c0 >> 7)];
      bfr = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(f[0] * sc, f[1] * sc), pack_bf16x2(f[2] * sc, f[3] * sc),
                                                  pack_bf16x2(f[4] * sc, f[5] * sc), pack_bf16x2(f[6] * sc, f[7] * sc)));
    }
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const int j = 16 * jt + L, ch = 4 * ks + g4;
      const bf16x8 wfr = *(const bf16x8*)(sw + j * 512 + ((ch ^ (j & 15)) << 3));
      acc[jt] = mfma16(wfr, bfr, acc[jt]);
    }
  }
  // lane: row bq, j = 16 jt + 4 g4 + 0..3
  float v[8][4];
  float amax = 0.f;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[jt][r] = __uint_as_float((uint32_t)f2bf(acc[jt][r]) << 16);
      amax = fmaxf(amax, fabsf(v[jt][r]));
    }
  if (a.o) {   // through LDS: [64 rows][128 j] bf16, 16-byte chunk k of row r at k ^ (r & 15)
    __syncthreads();   // every wave is done reading W_UV_h
    const int r = 16 * wave + L;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const int k = 2 * jt + (g4 >> 1);
      *(uint2*)(sw + r * 128 + ((k ^ (r & 15)) << 3) + 4 * (g4 & 1)) =
          make_uint2(pack_bf16x2(v[jt][0], v[jt][1]), pack_bf16x2(v[jt][2], v[jt][3]));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // pass i: rows 16 i + tid / 16, chunk tid % 16
      const int rr = 16 * i + (tid >> 4), k = tid & 15;
      if (b0 + rr < a.B)
        *(uint4*)((uint16_t*)a.o + (int64_t)(b0 + rr) * a.ldo + 128 * h + 8 * k) =
            *(const uint4*)(sw + rr * 128 + ((k ^ (rr & 15)) << 3));
    }
  }
  if (!row_ok) return;
  if (a.oq) {   // one 1x128 group per (row, head): lanes L, L + 16, L + 32, L + 48 hold it
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    e4m3_quotients(amax, true, [&](const float sc, auto quo) {
      uint8_t* q = a.oq + (int64_t)bq * a.ldo + 128 * h + 4 * g4;
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        uint32_t code = 0u;
        if (sc != 0.f)
          code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
              quo(v[jt][2]), quo(v[jt][3]), __builtin_amdgcn_cvt_pk_fp8_f32(quo(v[jt][0]), quo(v[jt][1]), 0, false),
              true);
        *(uint32_t*)(q + 16 * jt) = code;
      }
      if (g4 == 0) a.os[(int64_t)bq * (a.ldo / 128) + h] = sc;
    });
  }
}

}  // namespace

hipError_t launch_decode_unabsorb(const UnabsorbArgs& a, hipStream_t s) {
  if (a.splits < 1 || a.splits > DECODE_MAX_SPLITS || (a.splits > 1 && !a.lse) || a.ldo % 128 ||
      (!a.o && !a.oq) || (a.oq && !a.os))
    return hipErrorInvalidValue;
  dim3 grid(a.H, (a.B + 63) / 64);
  decode_unabsorb_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
