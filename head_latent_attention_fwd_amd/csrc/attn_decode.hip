// Latent-absorbed single-token decode attention (DeepSeek-V3.2-Exp · Sparse
// attention, "Explanation": a single decoded token scores the cached latent
// directly; DeepSeek-V3.2-Exp · Output projection page at p = 1000).
//
// With kv_b's key half folded into the query, every head of sequence b scores
// the same cache rows C_t = [latent 512 | rope key 64]:
//   z[h, t] = scale * (q_lat[h] . C_t),  o_lat[h] = sum_t softmax_t(z[h]) C_t[:512]
// so the cache is streamed from HBM once per sequence and shared by all heads.
//
// One 256-thread workgroup per (64-head group, sequence); wave w owns 16 heads.
// Scores are formed transposed (S^T = C . Q^T) on v_mfma_f32_16x16x32_bf16 so
// a lane holds 8 keys of one head; o_lat^T = C^T . P^T reuses the
// probabilities in place. Each 32-key tile is loaded once into LDS row-major
// (A operand of the scores) and transposed (A operand of the output), the
// transpose done as 8x8 register blocks.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int DKT = 32;        // keys per tile
constexpr int CP = 576 + 8;    // sC pitch (elements)
constexpr int TP = DKT + 4;    // sCt pitch (elements): conflict-free 8-byte reads

__device__ __forceinline__ uint32_t sel_lo(uint32_t a_hi, uint32_t b_lo) { return (a_hi << 16) | (b_lo & 0xFFFFu); }
__device__ __forceinline__ uint32_t sel_hi(uint32_t a_hi, uint32_t b_lo) { return (a_hi & 0xFFFF0000u) | (b_lo >> 16); }

__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sC[DKT * CP];
  __shared__ __attribute__((aligned(16))) uint16_t sCt[512 * TP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int hg = blockIdx.x, b = blockIdx.y, H = a.H;
  const int head = hg * 64 + wave * 16 + l16;
  const int P = a.cache_len[b];
  const bool ok = P >= 0 && P < a.max_len;
  const int nkeys = ok ? P + 1 : 0;

  bf16x8 qf[18];
  {
    const uint16_t* qp = (const uint16_t*)a.qlat + ((int64_t)b * H + head) * 576 + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + kk * 32));
  }
  floatx4 o[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const uint16_t* C = (const uint16_t*)a.cache + (int64_t)b * a.max_len * 576;

  const int kg = tid & 3, cblk = tid >> 2;   // transpose block: keys 8kg.., latent dims 8cblk..
  const int ntiles = (nkeys + DKT - 1) / DKT;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * DKT;
    uint4 rv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = k0 + kg * 8 + e;
      rv[e] = t < nkeys ? *(const uint4*)(C + (int64_t)t * 576 + cblk * 8) : make_uint4(0, 0, 0, 0);
    }
    {  // rope-key part of the tile: 32 keys x 8 chunks, one chunk per thread
      const int key = tid >> 3, part = 64 + (tid & 7), t = k0 + key;
      const uint4 v = t < nkeys ? *(const uint4*)(C + (int64_t)t * 576 + part * 8) : make_uint4(0, 0, 0, 0);
      *(uint4*)&sC[key * CP + part * 8] = v;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) *(uint4*)&sC[(kg * 8 + e) * CP + cblk * 8] = rv[e];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ((const uint32_t*)&rv[2 * j])[d >> 1];
        const uint32_t hi2 = ((const uint32_t*)&rv[2 * j + 1])[d >> 1];
        w[j] = (d & 1) ? sel_hi(hi2, lo) : sel_lo(hi2, lo);
      }
      uint16_t* dst = &sCt[(cblk * 8 + d) * TP + kg * 8];
      *(uint2*)dst = make_uint2(w[0], w[1]);
      *(uint2*)(dst + 4) = make_uint2(w[2], w[3]);
    }
    __syncthreads();

    floatx4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const bf16x8 cf = *(const bf16x8*)&sC[(kb * 16 + l16) * CP + kk * 32 + 8 * g];
        s[kb] = mfma16(cf, qf[kk], s[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = k0 + kb * 16 + 4 * g + r;
        const float v = t < nkeys ? s[kb][r] * sl2 : -INFINITY;
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m - muse);
    float rs = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2f(s[e >> 2][e & 3] - muse);
      rs += p;
      pf[e] = (__bf16)p;
    }
    l = l * alpha + rs;
    m = mnew;
    // keys of slot e: 16*(e/4) + 4g + e%4
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const uint16_t* vp = &sCt[(cb * 16 + l16) * TP + 4 * g];
      const uint2 lo = *(const uint2*)vp, hi2 = *(const uint2*)(vp + 16);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi2.x, hi2.y));
      o[cb] = mfma16(vf, pf, o[cb] * alpha);
    }
    __syncthreads();
  }

  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint16_t* op = (uint16_t*)a.olat + ((int64_t)b * H + head) * 512 + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    const uint2 pk = make_uint2(pack_bf16x2(o[cb][0] * inv, o[cb][1] * inv),
                                pack_bf16x2(o[cb][2] * inv, o[cb][3] * inv));
    *(uint2*)(op + cb * 16) = pk;
  }
}

}  // namespace

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s) {
  dim3 grid(a.H / 64, a.B);
  decode_attn_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
