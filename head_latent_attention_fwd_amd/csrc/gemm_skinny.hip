// Skinny bf16 GEMM for the decode step (M = batch <= 128 rows): C = A . W^T,
// bound by streaming W from HBM. One workgroup owns all M rows, NT columns of
// W and one K chunk (split-K over gridDim.y); every byte of W is read once and
// the small A chunk is re-read from L2. NT is 64, 96 or 128 columns. K moves
// in 64-wide steps through a 4-stage LDS ring of 16-byte direct-to-LDS loads
// (three steps in flight ahead of the MFMAs); chunks of each 128-byte row are XOR-swizzled by
// (row ^ row >> 3) & 7. Wave w computes rows 32w..32w+31 with
// v_mfma_f32_32x32x16_bf16 (W as the first operand, so a lane's results are 4
// consecutive columns of one row). With one split the bf16 result is stored
// directly; otherwise fp32 partials go to P[split][M][N] and are summed in a
// fixed order by splitk_reduce (or by the consumer), so results are
// deterministic.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int SK_BK = 64, SK_ST = 4;

__device__ __forceinline__ int sk_sw(int row) { return (row ^ (row >> 3)) & 7; }

// s_waitcnt lgkmcnt(0) and vmcnt(N), then a workgroup barrier
template <int N>
__device__ __forceinline__ void sk_wait_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ST-stage ring (ST - 1 steps in flight ahead of the MFMAs)
template <int NT, int ST>
__device__ __forceinline__ void gemm_skinny_body(const SkinnyArgs& g) {
  constexpr int SLOTS = (128 + NT) * 8;          // 16-byte slots per stage
  constexpr int LPT = SLOTS / 256;               // loads per thread per stage
  constexpr int STAGE = SLOTS * 8;               // elements per stage
  constexpr int FN = NT / 32;
  static_assert(SLOTS % 256 == 0 && NT % 32 == 0 && (ST == 3 || ST == 4) && (ST - 1) * LPT < 64, "ring shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[ST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int n0 = blockIdx.x * NT, split = blockIdx.y, z = blockIdx.z;
  const int M = g.M, N = g.N;
  const int k_begin = split * g.kc, k_end = min(g.K, k_begin + g.kc);
  const int nk = (k_end - k_begin) / SK_BK;
  const uint16_t* A = (const uint16_t*)g.A + (int64_t)z * g.batch_a + k_begin;
  const uint16_t* W = (const uint16_t*)g.W + (int64_t)z * g.batch_w + k_begin;
  const uint16_t* W2 = (const uint16_t*)g.W2 + k_begin;

  // slot p of a stage: rows 0..127 of A, then rows 0..NT-1 of W, 8 chunks each
  const uint16_t* src[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int p = (wave * LPT + i) * 64 + lane;
    const int r = p >> 3;
    if (p < 1024) {
      const int c = (p & 7) ^ sk_sw(r);
      src[i] = A + (int64_t)min(r, M - 1) * g.lda + c * 8;
    } else {
      const int rw = r - 128, c = (p & 7) ^ sk_sw(rw);
      const int n = min(n0 + rw, N - 1);
      src[i] = (n < g.n_split ? W + (int64_t)n * g.ldw : W2 + (int64_t)(n - g.n_split) * g.ldw2) + c * 8;
    }
  }
  auto issue = [&](int kt) {
    uint16_t* st = smem + (kt % ST) * STAGE + wave * LPT * 512;
#pragma unroll
    for (int i = 0; i < LPT; ++i) __builtin_amdgcn_global_load_lds(src[i] + kt * SK_BK, st + i * 512, 16, 0, 0);
  };
  // wait until step kt has landed; `ahead` (< ST) later steps may still be in flight
  auto wait_ahead = [&](int ahead) {
    if (ST == 4 && ahead >= 3) sk_wait_barrier<(ST - 1) * LPT>();
    else if (ahead >= 2) sk_wait_barrier<2 * LPT>();
    else if (ahead == 1) sk_wait_barrier<LPT>();
    else sk_wait_barrier<0>();
  };

  floatx16 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // swizzled offsets: A row 32 wave + l32 (parity of wave), W row 32 j + l32 (parity of j)
  int xa[4], xw[2][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    xa[kk] = ((2 * kk + hi) ^ sk_sw(32 * wave + l32)) << 3;
    xw[0][kk] = ((2 * kk + hi) ^ sk_sw(l32)) << 3;
    xw[1][kk] = ((2 * kk + hi) ^ sk_sw(32 + l32)) << 3;
  }
  bf16x8 fa[2], fb[2][FN];
  auto read = [&](int kt, int kk, int buf) {
    const uint16_t* st = smem + (kt % ST) * STAGE;
    fa[buf] = *(const bf16x8*)(st + (32 * wave + l32) * SK_BK + xa[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(st + (128 + 32 * j + l32) * SK_BK + xw[j & 1][kk]);
  };

  if (nk > 0) {
    for (int s = 0; s < ST; ++s)
      if (s < nk) issue(s);
    wait_ahead(min(nk, ST) - 1);   // step 0 has landed
  }
  if (nk > 0) read(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1;
      if (kk < 3) {
        read(kt, kk + 1, cb ^ 1);
      } else if (kt + 1 < nk) {
        wait_ahead(min(nk - 2 - kt, ST - 2));
        if (kt + ST < nk) issue(kt + ST);
        read(kt + 1, 0, cb ^ 1);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[j] = mfma32(fb[cb][j], fa[cb], acc[j]);
    }
  }

  // lane: row m = 32 wave + l32, columns n0 + 32 j + 8 rg + 4 hi + 0..3
  const int m = 32 * wave + l32;
  if (m >= M) return;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int n = n0 + 32 * j + 8 * rg + 4 * hi;
      if (n >= N) continue;
      const float v0 = acc[j][4 * rg], v1 = acc[j][4 * rg + 1], v2 = acc[j][4 * rg + 2], v3 = acc[j][4 * rg + 3];
      if (gridDim.y == 1) {
        uint16_t* c = (uint16_t*)g.C + (int64_t)z * g.batch_c + (int64_t)m * g.ldc + n;
        if (n + 4 <= N && (g.ldc & 3) == 0 && (g.batch_c & 3) == 0) {
          *(uint2*)c = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        } else {
          const float v[4] = {v0, v1, v2, v3};
          for (int e = 0; n + e < N; ++e) c[e] = f2bf(v[e]);
        }
      } else {
        float* p = g.P + (int64_t)split * g.ps + (int64_t)m * N + n;
        if (n + 4 <= N && (N & 3) == 0) {
          *(float4*)p = make_float4(v0, v1, v2, v3);
        } else {
          const float v[4] = {v0, v1, v2, v3};
          for (int e = 0; n + e < N; ++e) p[e] = v[e];
        }
      }
    }
}

// e4m3 x e4m3 variant: a 64-element bf16 step of the body above is one
// 128-byte K block here (one scale group), staged through the same ring as
// 16-byte chunks. Per block a wave runs two v_mfma_f32_32x32x64_f8f6f4 per
// 32-column group into a block accumulator that is then added to the running
// sum times a_scale[m, kb] * w_scale[n / 128, kb] (a lane's results share one
// row m, and a tile of at most 128 columns lies in one scale block). The
// scales of the workgroup's K chunk (at most SKF_KB blocks) are staged in LDS
// before the ring starts, so the ring's wait counts see only its own loads.
constexpr int SKF_KB = 32;
template <int NT>
__device__ __forceinline__ void gemm_skinny_fp8_body(const SkinnyArgs& g) {
  constexpr int SLOTS = (128 + NT) * 8;
  constexpr int LPT = SLOTS / 256;
  constexpr int STAGE = SLOTS * 8;               // uint16 units per stage
  constexpr int FN = NT / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SK_ST * STAGE];
  __shared__ float sa_s[128][SKF_KB + 1];
  __shared__ float sw_s[SKF_KB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int n0 = blockIdx.x * NT, split = blockIdx.y, z = blockIdx.z;
  const int M = g.M, N = g.N;
  const int k_begin = split * g.kc, k_end = min(g.K, k_begin + g.kc);
  const int nk = (k_end - k_begin) / 128;
  {  // scales of this chunk: rows of A, the tile's weight block row
    const int kb0 = k_begin / 128;
    const float* wsr = n0 < g.n_split ? g.ws + z * g.batch_ws + (int64_t)(n0 / 128) * g.ldws + kb0
                                      : g.ws2 + (int64_t)((n0 - g.n_split) / 128) * g.ldws + kb0;
    for (int i = tid; i < 128 * nk; i += 256) {
      const int r = i / nk, kb = i - r * nk;
      sa_s[r][kb] = g.as[z * g.batch_as + (int64_t)min(r, M - 1) * g.lds + kb0 + kb];
    }
    if (tid < nk) sw_s[tid] = wsr[tid];
  }
  // byte strides halved: the ring moves uint16 pairs
  const uint16_t* A = (const uint16_t*)((const uint8_t*)g.A + z * g.batch_a + k_begin);
  const uint16_t* W = (const uint16_t*)((const uint8_t*)g.W + z * g.batch_w + k_begin);
  const uint16_t* W2 = (const uint16_t*)((const uint8_t*)g.W2 + k_begin);
  const int64_t lda = g.lda / 2, ldw = g.ldw / 2, ldw2 = g.ldw2 / 2;

  const uint16_t* src[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int p = (wave * LPT + i) * 64 + lane;
    const int r = p >> 3;
    if (p < 1024) {
      const int c = (p & 7) ^ sk_sw(r);
      src[i] = A + (int64_t)min(r, M - 1) * lda + c * 8;
    } else {
      const int rw = r - 128, c = (p & 7) ^ sk_sw(rw);
      const int n = min(n0 + rw, N - 1);
      src[i] = (n < g.n_split ? W + (int64_t)n * ldw : W2 + (int64_t)(n - g.n_split) * ldw2) + c * 8;
    }
  }
  // The ring's loads are written as asm so that the compiler does not order
  // every later LDS read behind them; wait_ahead's explicit counts order them.
  auto issue = [&](int kt) {
    const uint32_t st = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(
        smem + (kt % SK_ST) * STAGE + wave * LPT * 512);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const uint32_t base = __builtin_amdgcn_readfirstlane(st + i * 1024);
      __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                       :
                       : "v"(src[i] + kt * SK_BK), "s"(base)
                       : "memory", "m0");
    }
  };
  auto wait_ahead = [&](int ahead) {
    if (ahead >= 3) {
      if constexpr (LPT == 6) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(18)" ::: "memory");
      else __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(24)" ::: "memory");
    } else if (ahead == 2) {
      if constexpr (LPT == 6) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(12)" ::: "memory");
      else __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(16)" ::: "memory");
    } else if (ahead == 1) {
      if constexpr (LPT == 6) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(6)" ::: "memory");
      else __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(8)" ::: "memory");
    } else {
      __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };

  floatx16 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // a lane's 32 k bytes of sub-step s are chunks 4 s + 2 hi and 4 s + 2 hi + 1
  const int ra = 32 * wave + l32;
  int xa[2][2], xw[2][2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 4 * s + 2 * hi + e;
      xa[s][e] = (ch ^ sk_sw(ra)) << 3;
      xw[0][s][e] = (ch ^ sk_sw(l32)) << 3;
      xw[1][s][e] = (ch ^ sk_sw(32 + l32)) << 3;
    }
  auto frag = [&](const uint16_t* row, const int* x) {
    const intx4 lo = __builtin_bit_cast(intx4, *(const bf16x8*)(row + x[0]));
    const intx4 up = __builtin_bit_cast(intx4, *(const bf16x8*)(row + x[1]));
    return (intx8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
  };

  const int m = ra;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the scale loads, before the ring's
  // fragments of one step: A (two 32-byte sub-steps) and W per column group
  intx8 af[2], wf[2][FN];
  auto read = [&](int kt) {
    const uint16_t* st = smem + (kt % SK_ST) * STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      af[s] = frag(st + ra * SK_BK, xa[s]);
#pragma unroll
      for (int j = 0; j < FN; ++j) wf[s][j] = frag(st + (128 + 32 * j + l32) * SK_BK, xw[j & 1][s]);
    }
  };
  // a_scale[m, kb] * w_scale[kb] of step kb, read from LDS in an asm block
  // that waits for its own reads: the compiler would otherwise order these
  // reads behind every load of the ring still in flight
  auto scale = [&](int kb) {
    const uint32_t pa = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&sa_s[m][kb];
    const uint32_t pw = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&sw_s[kb];
    float a, w;
    __asm__ volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(a), "=&v"(w)
                     : "v"(pa), "v"(pw)
                     : "memory");
    return a * w;
  };
  // Software-pipelined over two block accumulators: step kt + 1's MFMAs are
  // issued before step kt's block is added to the running sum, so those 16 FMAs
  // per block run on the VALU while the matrix core works on the next step.
  auto mfmas = [&](floatx16* blk) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      floatx16 zero;
#pragma unroll
      for (int r = 0; r < 16; ++r) zero[r] = 0.f;
      blk[j] = mfma32_fp8(wf[0][j], af[0], zero);
      blk[j] = mfma32_fp8(wf[1][j], af[1], blk[j]);
    }
  };
  auto promote = [&](const floatx16* blk, float fc) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = fmaf(blk[j][r], fc, acc[j][r]);
  };
  float f = 0.f;
  // step kt + 1 has landed and every wave is done with stage kt, which is
  // refilled; then step kt + 1's fragments and scale are read
  auto advance = [&](int kt) __attribute__((always_inline)) {
    wait_ahead(min(nk - 2 - kt, 2));
    if (kt + SK_ST < nk) issue(kt + SK_ST);
    f = scale(kt + 1);
    read(kt + 1);
  };
  if (nk > 0) {
    for (int s = 0; s < SK_ST; ++s)
      if (s < nk) issue(s);
    wait_ahead(min(nk, SK_ST) - 1);   // step 0 (and the staged scales) have landed
    read(0);
    f = scale(0);
    floatx16 b0[FN], b1[FN];
    mfmas(b0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {   // b0 holds step kt's products, f its scale
      float fc = f;
      advance(kt);
      mfmas(b1);
      promote(b0, fc);
      fc = f;
      if (kt + 2 < nk) {
        advance(kt + 1);
        mfmas(b0);
      }
      promote(b1, fc);
    }
    if (kt < nk) promote(b0, f);
  }

  if (NT == 128 && g.qc) {
    // e4m3 output: the row's 128 columns are this lane's 64 values and those
    // of lane ^ 32; quantised from their bf16 values (rows past M idle along)
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[j][r] = __uint_as_float((uint32_t)f2bf(acc[j][r]) << 16);
        amax = fmaxf(amax, fabsf(acc[j][r]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (m >= M) return;
    uint8_t* qrow = g.qc + (int64_t)m * g.ldc + (int64_t)z * g.batch_c;
    e4m3_quotients(amax, true, [&](const float s, auto quo) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float v0 = acc[j][4 * rg], v1 = acc[j][4 * rg + 1], v2 = acc[j][4 * rg + 2], v3 = acc[j][4 * rg + 3];
          uint32_t code = 0u;
          if (s != 0.f)
            code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                quo(v2), quo(v3), __builtin_amdgcn_cvt_pk_fp8_f32(quo(v0), quo(v1), 0, false), true);
          *(uint32_t*)(qrow + 32 * j + 8 * rg + 4 * hi) = code;
        }
      if (hi == 0) g.qs[(int64_t)m * (g.ldc / 128) + z * (g.batch_c / 128)] = s;
    });
    return;
  }
  if (m >= M) return;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int n = n0 + 32 * j + 8 * rg + 4 * hi;
      if (n >= N) continue;
      const float v0 = acc[j][4 * rg], v1 = acc[j][4 * rg + 1], v2 = acc[j][4 * rg + 2], v3 = acc[j][4 * rg + 3];
      if (gridDim.y == 1) {
        uint16_t* c = (uint16_t*)g.C + (int64_t)z * g.batch_c + (int64_t)m * g.ldc + n;
        if (n + 4 <= N && (g.ldc & 3) == 0 && (g.batch_c & 3) == 0) {
          *(uint2*)c = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        } else {
          const float v[4] = {v0, v1, v2, v3};
          for (int e = 0; n + e < N; ++e) c[e] = f2bf(v[e]);
        }
      } else {
        float* p = g.P + (int64_t)split * g.ps + (int64_t)m * N + n;
        if (n + 4 <= N && (N & 3) == 0) {
          *(float4*)p = make_float4(v0, v1, v2, v3);
        } else {
          const float v[4] = {v0, v1, v2, v3};
          for (int e = 0; n + e < N; ++e) p[e] = v[e];
        }
      }
    }
}

__global__ __launch_bounds__(256, 1) void gemm_skinny64_kernel(SkinnyArgs g) { gemm_skinny_body<64, 4>(g); }
__global__ __launch_bounds__(256, 1) void gemm_skinny96_kernel(SkinnyArgs g) { gemm_skinny_body<96, 4>(g); }
__global__ __launch_bounds__(256, 1) void gemm_skinny_fp8_64_kernel(SkinnyArgs g) { gemm_skinny_fp8_body<64>(g); }
__global__ __launch_bounds__(256, 1) void gemm_skinny_fp8_128_kernel(SkinnyArgs g) { gemm_skinny_fp8_body<128>(g); }
__global__ __launch_bounds__(256, 1) void gemm_skinny128_kernel(SkinnyArgs g) { gemm_skinny_body<128, 4>(g); }

// out[m, n] = sum over s of P[s][m][n] (s ascending), stored bf16.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* P, int S, int M, int N, uint16_t* out,
                                                            int64_t ldo) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  if (n + 4 <= N && (N & 3) == 0) {
    float4 acc = *(const float4*)(P + i);
    for (int s = 1; s < S; ++s) {
      const float4 v = *(const float4*)(P + (int64_t)s * total + i);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *(uint2*)(out + (int64_t)m * ldo + n) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  } else {
    for (int e = 0; e < 4 && i + e < total; ++e) {
      const int me = (int)((i + e) / N), ne = (int)((i + e) - (int64_t)me * N);
      float a = 0.f;
      for (int s = 0; s < S; ++s) a += P[(int64_t)s * total + i + e];
      out[(int64_t)me * ldo + ne] = f2bf(a);
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const SkinnyArgs& g, int nt, int splits, hipStream_t s) {
  dim3 grid((g.N + nt - 1) / nt, splits, g.batch);
  if (nt == 64) gemm_skinny64_kernel<<<grid, 256, 0, s>>>(g);
  else if (nt == 96) gemm_skinny96_kernel<<<grid, 256, 0, s>>>(g);
  else if (nt == 128) gemm_skinny128_kernel<<<grid, 256, 0, s>>>(g);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_skinny_fp8(const SkinnyArgs& g, int nt, int splits, hipStream_t s) {
  if (g.K % 128 || g.kc % 128 || g.lda % 16 || g.ldw % 16 || (g.W2 && (g.ldw2 % 16 || g.n_split % 128)) ||
      g.batch_a % 16 || g.batch_w % 16 || g.M > 128 || (nt != 64 && nt != 128) || g.kc > 128 * SKF_KB ||
      !g.as || !g.ws || (g.W2 && !g.ws2) ||
      (g.qc && (nt != 128 || g.N != 128 || splits != 1 || !g.qs || g.ldc % 128 || g.batch_c % 128)) ||
      (((uintptr_t)g.A | (uintptr_t)g.W | (uintptr_t)g.W2) & 15))
    return hipErrorInvalidValue;
  dim3 grid((g.N + nt - 1) / nt, splits, g.batch);
  if (nt == 64) gemm_skinny_fp8_64_kernel<<<grid, 256, 0, s>>>(g);
  else gemm_skinny_fp8_128_kernel<<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* P, int S, int M, int N, void* out, int64_t ldo, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  splitk_reduce_kernel<<<(unsigned)((total / 4 + 255) / 256 + 1), 256, 0, s>>>(P, S, M, N, (uint16_t*)out, ldo);
  return hipGetLastError();
}

}  // namespace mla
