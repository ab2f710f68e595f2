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
// ds_read_b64_tr_b16 and q read straight from global memory; a lane's results
// are 4 consecutive c of one sequence, stored as 8-byte pieces. Wave w covers
// c in [256 z + 128 (w & 1), +128) and sequences [32 (w >> 1), +32) of the tile.
// The q_pe rotation of the tile is split between the two halves by pair index.
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
  // ks, q_nope dims 16 ks + 4 hi + 0..3 and 16 ks + 8 + 4 hi + 0..3
  const int l32 = lane & 31, hi = lane >> 5, wc = wave & 1, wb = wave >> 1;
  const int bq = b0 + wb * 32 + l32;
  bf16x8 qf[8];
  {
    const uint16_t* qp = q + ((int64_t)min(bq, B - 1) * H + h) * 192 + 4 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint2 lo = *(const uint2*)(qp + 16 * ks), up = *(const uint2*)(qp + 16 * ks + 8);
      qf[ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, up.x, up.y));
    }
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

  // W^T fragments: 16-lane group g reads rows j = 16 ks + 4 (g >> 1) + 8 e + (lane % 16) / 4,
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
      const int j0 = 16 * ks + 4 * (g >> 1) + (L >> 2), j1 = j0 + 8;
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
  if (bq < B) {
    uint16_t* o = qlat + ((int64_t)bq * H + h) * 576 + 256 * z + 128 * wc + 4 * hi;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *(uint2*)(o + 32 * cb + 8 * rg) = make_uint2(pack_bf16x2(acc[cb][4 * rg], acc[cb][4 * rg + 1]),
                                                     pack_bf16x2(acc[cb][4 * rg + 2], acc[cb][4 * rg + 3]));
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
