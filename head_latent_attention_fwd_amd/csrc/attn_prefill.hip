// Fused MLA prefill attention (DeepSeek-V3.2-Exp · Sparse attention, "Code":
// per head, scores = scale * [q_nope | q_pe] . [k_nope | shared k_pe], the
// selection and causal masks, softmax over keys, then the weighted sum of
// values). The T x T score matrix is never written: keys are streamed in
// 64-key tiles with an online softmax.
//
// Work split: one 256-thread workgroup per (128-query tile, head, sequence);
// wave w owns queries [32w, 32w+32) of the tile. Scores are formed transposed,
// S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16 so that a lane holds 32 keys of a
// single query: the running max needs one cross-lane exchange (lane ^ 32) and
// the running sum stays lane-local. The probabilities, rounded to bf16, are
// already in the B-operand layout of O^T = V^T . P^T. Q stays in registers as
// the B operand; the K tile is stored row-major in LDS, the V tile transposed
// (8x8 register transposes, 8-byte LDS stores).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BQ = 128;       // queries per workgroup
constexpr int BKV = 64;       // keys per tile
constexpr int KP = 192 + 8;   // sK pitch (elements): 400 B, conflict-free 16-B reads
constexpr int VP = BKV + 4;   // sVt pitch (elements): 136 B, conflict-free 8-B reads

__device__ __forceinline__ uint32_t sel_lo(uint32_t a_hi, uint32_t b_lo) {  // (a.lo16 << 16) | b.lo16
  return (a_hi << 16) | (b_lo & 0xFFFFu);
}
__device__ __forceinline__ uint32_t sel_hi(uint32_t a_hi, uint32_t b_lo) {  // (a.hi16 << 16) | b.hi16
  return (a_hi & 0xFFFF0000u) | (b_lo >> 16);
}

__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BKV * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[128 * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, H = a.H;
  const int64_t ldq = (int64_t)H * 192, ldu = (int64_t)H * 256, ldo = (int64_t)H * 128;
  const int64_t row0 = (int64_t)b * T;
  const uint16_t* Q = (const uint16_t*)a.q;
  const uint16_t* U = (const uint16_t*)a.u;
  const uint16_t* KV = (const uint16_t*)a.kv;
  const int q0 = qt * BQ, qw = q0 + wave * 32;
  const int l32 = lane & 31, hi = lane >> 5;

  // Q^T operand: lane holds query qw + l32, dims 16*kk + 8*hi + 0..7.
  const int qi = qw + l32;
  const bool q_ok = qi < T;
  bf16x8 qf[12];
  {
    const uint16_t* qp = Q + (row0 + (q_ok ? qi : 0)) * ldq + h * 192 + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
      uint4 v = q_ok ? *(const uint4*)(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  floatx16 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int W = (T + 31) >> 5;
  const uint32_t* mrow = a.mask ? a.mask + (row0 + (q_ok ? qi : 0)) * W : nullptr;

  const int kv_end = min(T, q0 + BQ);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BKV;
    // K tile: [k_nope (from u) | k_pe (from kv)] per key, 24 chunks of 8.
    for (int c = tid; c < BKV * 24; c += 256) {
      const int key = c / 24, part = c - key * 24, t = k0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < T) {
        v = part < 16 ? *(const uint4*)(U + (row0 + t) * ldu + h * 256 + part * 8)
                      : *(const uint4*)(KV + (row0 + t) * a.ld_kv + a.kpe_off + (part - 16) * 8);
      }
      *(uint4*)&sK[key * KP + part * 8] = v;
    }
    // V tile transposed: thread < 128 owns keys 8*kg..8*kg+7 x dims 8*db..8*db+7.
    if (tid < 128) {
      const int kg = tid & 7, db = tid >> 3;
      uint4 rv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = k0 + kg * 8 + e;
        rv[e] = t < T ? *(const uint4*)(U + (row0 + t) * ldu + h * 256 + 128 + db * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = ((const uint32_t*)&rv[2 * j])[d >> 1];
          const uint32_t hi2 = ((const uint32_t*)&rv[2 * j + 1])[d >> 1];
          w[j] = (d & 1) ? sel_hi(hi2, lo) : sel_lo(hi2, lo);
        }
        uint16_t* dst = &sVt[(db * 8 + d) * VP + kg * 8];
        *(uint2*)dst = make_uint2(w[0], w[1]);
        *(uint2*)(dst + 4) = make_uint2(w[2], w[3]);
      }
    }
    __syncthreads();

    if (k0 <= qw + 31) {
      floatx16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 12; ++kk) {
          const bf16x8 kf = *(const bf16x8*)&sK[(kb * 32 + l32) * KP + kk * 16 + hi * 8];
          s[kb] = mfma32(kf, qf[kk], s[kb]);
        }
      }
      // mask + scale (log2 domain); lane holds keys k0 + 32kb + row32(r)
      uint32_t mw0 = 0xFFFFFFFFu, mw1 = 0xFFFFFFFFu;
      if (mrow) {
        mw0 = mrow[k0 >> 5];
        mw1 = ((k0 >> 5) + 1 < W) ? mrow[(k0 >> 5) + 1] : 0u;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = row32(r, lane);
          const int t = k0 + kb * 32 + kr;
          const uint32_t bits = kb ? mw1 : mw0;
          const bool live = t <= qi && t < T && ((bits >> kr) & 1u);
          const float v = live ? s[kb][r] * sl2 : -INFINITY;
          s[kb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m - muse);
      float rs = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = exp2f(s[kb][half * 8 + e] - muse);
            rs += p;
            pf[kb * 2 + half][e] = (__bf16)p;
          }
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      // O^T += V^T . P^T; k-step ks covers keys 32kb + 16half + {8(e/4) + 4hi + e%4}
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int base = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* vp = &sVt[(j * 32 + l32) * VP + base];
          const uint2 lo = *(const uint2*)vp, hi2 = *(const uint2*)(vp + 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi2.x, hi2.y));
          o[j] = mfma32(vf, pf[ks], o[j]);
        }
      }
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (q_ok) {
    uint16_t* op = (uint16_t*)a.out + (row0 + qi) * ldo + h * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int dv = j * 32 + row32(r, lane);
        uint2 pk = make_uint2(pack_bf16x2(o[j][r] * inv, o[j][r + 1] * inv),
                              pack_bf16x2(o[j][r + 2] * inv, o[j][r + 3] * inv));
        *(uint2*)(op + dv) = pk;
      }
  }
}

// fp32 path: one wave per (query, head); lanes split the feature dims.
__global__ __launch_bounds__(64) void prefill_attn_f32_kernel(PrefillAttnArgs a) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int T = a.T, H = a.H;
  const int64_t row0 = (int64_t)b * T;
  const float* Q = (const float*)a.q + (row0 + s) * H * 192 + h * 192;
  const float* U = (const float*)a.u;
  const float* KV = (const float*)a.kv;
  const float q0 = Q[lane], q1 = Q[lane + 64], q2 = Q[lane + 128];
  const int W = (T + 31) >> 5;
  const uint32_t* mrow = a.mask ? a.mask + (row0 + s) * W : nullptr;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t = 0; t <= s; ++t) {
    if (mrow && !((mrow[t >> 5] >> (t & 31)) & 1u)) continue;
    const float* ut = U + (row0 + t) * H * 256 + h * 256;
    const float* kp = KV + (row0 + t) * a.ld_kv + a.kpe_off;
    float d = q0 * ut[lane] + q1 * ut[lane + 64] + q2 * kp[lane];
    d = wave_sum(d) * a.scale;
    const float mn = fmaxf(m, d);
    const float al = expf(m - mn), p = expf(d - mn);
    l = l * al + p;
    o0 = o0 * al + p * ut[128 + lane];
    o1 = o1 * al + p * ut[128 + lane + 64];
    m = mn;
  }
  float* op = (float*)a.out + (row0 + s) * H * 128 + h * 128;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  op[lane] = o0 * inv;
  op[lane + 64] = o1 * inv;
}

}  // namespace

hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, hipStream_t s) {
  dim3 grid((a.T + BQ - 1) / BQ, a.H, a.B);
  prefill_attn_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_f32(const PrefillAttnArgs& a, hipStream_t s) {
  dim3 grid(a.T, a.H, a.B);
  prefill_attn_f32_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
