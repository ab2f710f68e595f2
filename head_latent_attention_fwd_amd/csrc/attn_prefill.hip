// Fused MLA prefill attention (DeepSeek-V3.2-Exp · Sparse attention, "Code":
// per head, scores = scale * [q_nope | q_pe] . [k_nope | shared k_pe], the
// selection and causal masks, softmax over keys, then the weighted sum of
// values). The T x T score matrix is never written: keys are streamed in
// 64-key tiles with an online softmax.
//
// Inputs are laid out for streaming: k_nope per head [B, H, Tp, 128], the
// values per head already transposed [B, H, 128, Tp] (both written so by the
// kv_b GEMM's epilogue) and the shared rotary key [B, Tp, 64].
//
// Work split: one 256-thread workgroup per (128-query tile, head, sequence),
// heaviest (last) query tiles first; wave w owns queries [32w, 32w+32).
// Scores are formed transposed, S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16 so
// a lane holds 32 keys of one query: the running max needs one exchange
// (lane ^ 32) and the running sum stays lane-local; the bf16 probabilities are
// the B operand of O^T = V^T . P^T. Q stays in registers.
//
// Tiles move HBM -> LDS with gfx950's 16-byte direct-to-LDS loads into a
// two-stage ring (one barrier per tile; the next tile's loads fly while the
// current tile is consumed), 40 KB per stage, two workgroups per CU. Within a
// 16-key block the K rows are stored with bits 2 and 3 of the key index
// swapped: the 32x32 MFMA output then gives each lane 8 consecutive keys per
// 16-key step, so the matching V^T operand is one 16-byte LDS read. 16-byte
// chunks are XOR-swizzled by row in every region (conflict-free reads with 32
// or 64 LDS banks).
//
// The running max is only raised when a row's max grows by more than 2^8
// (probabilities stay <= 256 in the meantime), so the O rescale is rare.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BQ = 128;                   // queries per workgroup
constexpr int BKV = 64;                   // keys per tile
// one LDS stage (bf16 elements): k_nope [64][128] | k_pe [64][64] | v^T [128][64]
constexpr int ST_KN = 0, ST_KPE = 64 * 128, ST_VT = ST_KPE + 64 * 64, STAGE = ST_VT + 128 * 64;
constexpr int LOADS = STAGE * 2 / 16 / 256;  // 16-byte direct loads per thread per tile (10)
constexpr float LAZY = 8.0f;

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// chunk swizzle of 128-byte rows, conflict-free for 32 or 64 LDS banks
__device__ __forceinline__ int sw8(int r) { return (r ^ (r >> 3)) & 7; }

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int T = a.T, Tp = a.Tp, H = a.H;
  const int qt = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  const int q0 = qt * BQ, qw = q0 + wave * 32;
  const int qi = qw + l32;
  const bool q_ok = qi < T;

  bf16x8 qf[12];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)b * T + (q_ok ? qi : 0)) * ((int64_t)H * 192) + h * 192 + hi * 8;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
      const uint4 v = q_ok ? *(const uint4*)(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Direct-load slots: wave w fills 1 KB blocks LOADS*w .. LOADS*w + LOADS-1 of a
  // stage; lane l of block i lands in 16-byte slot p = 64 i + l.
  const uint16_t* src[LOADS];
  int adv[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = (wave * LOADS + i) * 64 + lane;
    if (p < ST_KPE / 8) {                       // k_nope: row rho, chunk' = chunk ^ (rho & 15)
      const int rho = p >> 4, c = (p & 15) ^ (rho & 15);
      src[i] = (const uint16_t*)a.kn + (bh * Tp + swap23(rho)) * 128 + c * 8;
      adv[i] = BKV * 128;
    } else if (p < ST_VT / 8) {                 // k_pe
      const int q = p - ST_KPE / 8, rho = q >> 3, c = (q & 7) ^ sw8(rho);
      src[i] = (const uint16_t*)a.kpe + ((int64_t)b * Tp + swap23(rho)) * 64 + c * 8;
      adv[i] = BKV * 64;
    } else {                                    // v^T: row dv, 8-key chunk
      const int q = p - ST_VT / 8, dv = q >> 3, c = (q & 7) ^ sw8(dv);
      src[i] = (const uint16_t*)a.vt + (bh * 128 + dv) * Tp + c * 8;
      adv[i] = BKV;
    }
  }
  auto issue = [&](int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      __builtin_amdgcn_global_load_lds(src[i], smem + stage * STAGE + (wave * LOADS + i) * 512, 16, 0, 0);
      src[i] += adv[i];
    }
  };

  // LDS operand offsets (elements), invariant over tiles
  const int x15 = l32 & 15;
  int xk[8], xp[2][4];
#pragma unroll
  for (int v = 0; v < 8; ++v) xk[v] = ((2 * v + hi) ^ x15) << 3;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 4; ++v) xp[kb][v] = ((2 * v + hi) ^ sw8(kb * 32 + l32)) << 3;

  floatx16 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int W = (T + 31) >> 5;
  const uint32_t* mrow = a.mask ? a.mask + ((int64_t)b * T + (q_ok ? qi : 0)) * W : nullptr;

  const int kv_end = min(T, q0 + BQ);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  issue(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1, k0 = kt * BKV;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < ntiles) issue(cur ^ 1);
    if (k0 > qw + 31) continue;                  // every key of the tile is after this wave's queries
    const uint16_t* sb = smem + cur * STAGE;
    uint32_t mw0 = 0xFFFFFFFFu, mw1 = 0xFFFFFFFFu;
    if (mrow) {
      mw0 = mrow[k0 >> 5];
      mw1 = ((k0 >> 5) + 1 < W) ? mrow[(k0 >> 5) + 1] : 0u;
    }
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 12; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int rho = kb * 32 + l32;
        const int off = kk < 8 ? ST_KN + rho * 128 + xk[kk] : ST_KPE + rho * 64 + xp[kb][kk - 8];
        s[kb] = mfma32(*(const bf16x8*)(sb + off), qf[kk], s[kb]);
      }
    }
    // s[kb][r] holds key k0 + 32kb + 16(r/8) + 8hi + r%8
    const bool interior = !mrow && (k0 + BKV - 1 <= qw) && (k0 + BKV <= T);
    if (!interior) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t bits = kb ? mw1 : mw0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 16 * (r >> 3) + 8 * hi + (r & 7);
          const int t = k0 + kb * 32 + kr;
          const bool live = t <= qi && t < T && ((bits >> kr) & 1u);
          s[kb][r] = live ? s[kb][r] : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    const bool raise = mx > m + LAZY;
    if (__any(raise)) {
      const float mn = raise ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);   // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] *= alpha;
      m = mn;
    }
    const float ms = m == -INFINITY ? 0.f : m;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][half * 8 + e], sl2, -ms));
          l += p;
          pf[kb * 2 + half][e] = (__bf16)p;
        }
    // O^T += V^T . P^T; step ks covers keys 32(ks/2) + 16(ks%2) + 8hi + 0..7
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dv = j * 32 + l32;
        const int c = (4 * (ks >> 1) + 2 * (ks & 1) + hi) ^ sw8(dv);
        const bf16x8 vf = *(const bf16x8*)(sb + ST_VT + dv * 64 + (c << 3));
        o[j] = mfma32(vf, pf[ks], o[j]);
      }
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (q_ok) {
    uint16_t* op = (uint16_t*)a.out + ((int64_t)b * T + qi) * ((int64_t)H * 128) + h * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int dv = j * 32 + row32(r, lane);
        const uint2 pk2 = make_uint2(pack_bf16x2(o[j][r] * inv, o[j][r + 1] * inv),
                                     pack_bf16x2(o[j][r + 2] * inv, o[j][r + 3] * inv));
        *(uint2*)(op + dv) = pk2;
      }
  }
}

// fp32 path: one wave per (query, head); lanes split the feature dims.
__global__ __launch_bounds__(64) void prefill_attn_f32_kernel(PrefillAttnArgs a) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int T = a.T, Tp = a.Tp, H = a.H;
  const int64_t bh = (int64_t)b * H + h;
  const float* Q = (const float*)a.q + ((int64_t)b * T + s) * H * 192 + h * 192;
  const float* KN = (const float*)a.kn + bh * Tp * 128;
  const float* VT = (const float*)a.vt + bh * 128 * Tp;
  const float* KP = (const float*)a.kpe + (int64_t)b * Tp * 64;
  const float q0 = Q[lane], q1 = Q[lane + 64], q2 = Q[lane + 128];
  const int W = (T + 31) >> 5;
  const uint32_t* mrow = a.mask ? a.mask + ((int64_t)b * T + s) * W : nullptr;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t = 0; t <= s; ++t) {
    if (mrow && !((mrow[t >> 5] >> (t & 31)) & 1u)) continue;
    float d = q0 * KN[t * 128 + lane] + q1 * KN[t * 128 + lane + 64] + q2 * KP[t * 64 + lane];
    d = wave_sum(d) * a.scale;
    const float mn = fmaxf(m, d);
    const float al = expf(m - mn), p = expf(d - mn);
    l = l * al + p;
    o0 = o0 * al + p * VT[(int64_t)lane * Tp + t];
    o1 = o1 * al + p * VT[(int64_t)(lane + 64) * Tp + t];
    m = mn;
  }
  float* op = (float*)a.out + ((int64_t)b * T + s) * H * 128 + h * 128;
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
