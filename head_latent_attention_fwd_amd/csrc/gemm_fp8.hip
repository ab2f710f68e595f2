// Block-scaled FP8 (OCP e4m3) GEMM on gfx950 (Kimi K2 · Down projection,
// quantization_config: e4m3 weights with one scale per 128 x 128 block and
// dynamically quantised activations).
//
//   C[m, n] = sum_g a_scale[m, g] * w_scale[n/128, g] * sum_{k in g} Aq[m, k] Wq[n, k]
//
// One K step is exactly one 128-wide scale group. The group's partial product
// is formed by two v_mfma_f32_32x32x64_f8f6f4 per 32x32 block into a fresh
// accumulator, then promoted into the fp32 result with the row's activation
// scale times the tile's weight scale (the scales are arbitrary fp32, so the
// MX e8m0 block-scale operands of the instruction do not apply). A and W tiles
// are staged through LDS (144-byte pitch), double-buffered.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BK = 128;       // bytes of K per step = one scale group
constexpr int LDB = BK + 16;  // LDS pitch in bytes

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(GemmFp8Args g) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * BK / 16 / 256;
  constexpr int WCH = BN * BK / 16 / 256;
  static_assert(BN == 128, "one weight-scale block per tile column range");
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDB];
  __shared__ __attribute__((aligned(16))) uint8_t sW[2][BN * LDB];
  __shared__ __attribute__((aligned(16))) float sAs[2][BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = g.M, N = g.N, K = g.K, KG = K / 128;

  const uint8_t* a_ptr[ACH];
  int a_lds[ACH];
  bool a_ok[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
    a_ok[i] = (m0 + row) < M;
    a_ptr[i] = g.A + (int64_t)(a_ok[i] ? m0 + row : 0) * K + col;
    a_lds[i] = row * LDB + col;
  }
  const uint8_t* w_ptr[WCH];
  int w_lds[WCH];
  bool w_ok[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16, n = n0 + row;
    w_ok[i] = n < N;
    int nn = w_ok[i] ? n : 0;
    w_ptr[i] = (nn < g.n_split ? g.W + (int64_t)nn * K : g.W2 + (int64_t)(nn - g.n_split) * K) + col;
    w_lds[i] = row * LDB + col;
  }
  // weight-scale row of this tile
  const float* wsc = n0 < g.n_split ? g.w_scale + (int64_t)(n0 / 128) * KG
                                    : g.w2_scale + (int64_t)((n0 - g.n_split) / 128) * KG;
  const bool as_ok = tid < BM && (m0 + tid) < M;
  const float* as_ptr = g.a_scale + (int64_t)(as_ok ? m0 + tid : 0) * KG;

  uint4 ra[ACH], rw[WCH];
  float ras = 0.f;
  auto load_global = [&](int kg) {
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[i] = a_ok[i] ? *(const uint4*)(a_ptr[i] + kg * BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < WCH; ++i)
      rw[i] = w_ok[i] ? *(const uint4*)(w_ptr[i] + kg * BK) : make_uint4(0, 0, 0, 0);
    ras = as_ok ? as_ptr[kg] : 0.f;
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(uint4*)&sA[buf][a_lds[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) *(uint4*)&sW[buf][w_lds[i]] = rw[i];
    if (tid < BM) sAs[buf][tid] = ras;
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_global(0);
  store_lds(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 32;
  for (int kg = 0; kg < KG; ++kg) {
    const int cur = kg & 1;
    const float sw = wsc[kg];
    if (kg + 1 < KG) load_global(kg + 1);
    floatx16 part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) part[i][j][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      intx8 af[FM], bw[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint8_t* p = &sA[cur][(wm * WM + i * 32 + lrow) * LDB + ks * 64 + lk];
        intx4 lo = *(const intx4*)p, hi = *(const intx4*)(p + 16);
        af[i] = (intx8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint8_t* p = &sW[cur][(wn * WN + j * 32 + lrow) * LDB + ks * 64 + lk];
        intx4 lo = *(const intx4*)p, hi = *(const intx4*)(p + 16);
        bw[j] = (intx8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) part[i][j] = mfma32_fp8(af[i], bw[j], part[i][j]);
    }
    // promote: acc += part * a_scale[row] * w_scale
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float srow[16];
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        floatx4 v = *(const floatx4*)&sAs[cur][wm * WM + i * 32 + row32(r, lane)];
        srow[r] = v[0] * sw; srow[r + 1] = v[1] * sw; srow[r + 2] = v[2] * sw; srow[r + 3] = v[3] * sw;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(part[i][j][r], srow[r], acc[i][j][r]);
    }
    if (kg + 1 < KG) store_lds(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WN + j * 32 + lrow;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WM + i * 32 + row32(r, lane);
        if (m >= M) continue;
        if (g.epi == EPI_KV_SPLIT)
          kv_split_store(g.kv, (uint16_t*)g.C, (uint16_t*)g.kv.vt, m, n, f2bf(acc[i][j][r]));
        else if (g.c_dtype == DT_F32)
          ((float*)g.C)[(int64_t)m * g.ldc + n] = acc[i][j][r];
        else
          ((uint16_t*)g.C)[(int64_t)m * g.ldc + n] = f2bf(acc[i][j][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Large-shape kernel: 256 x 256 tiles, eight waves as 4 x 2, each a 64 x 128
// block of v_mfma_f32_32x32x64_f8f6f4 results (W as the first operand, so a
// lane holds one output row and 4 consecutive columns per block row group).
// A wave's 128 columns are one weight-scale block, so the promotion scale of
// a lane's row in group g is one number s_g = a_scale[m, g] * w_scale[blk, g].
// Instead of a second accumulator per group, the running sum is kept in units
// of the latest scale: before group g's MFMAs it is multiplied by
// s_{g-1} / s_g, and the final sum by s_last, which telescopes to
// sum_g s_g P_g. A group with s_g = 0 has all-zero codes and leaves the sum
// and the running scale unchanged. The accumulators stay in VGPRs for that
// multiply; two waves per SIMD hide each other's LDS and MFMA latencies.
// K moves one 128-wide scale group per step through two LDS stages (64 KB
// each: 256 A rows then 256 W rows of 128 bytes, 16-byte chunks swizzled by
// (row >> 1) & 7) filled by 16-byte loads straight into LDS.
// Column tiles never straddle n_split (multiple of 128); output bf16 through
// LDS (row-major or the k_nope / v^T split).
//
// Two forms of the K loop. With many groups (wo, q_a||kv_a) the loads are
// raw-buffer builtins and the scales plain loads issued a step ahead. With
// few groups per tile (kv_b: 4, q_b: 12) a tile's time is dominated by its
// first groups' trips to HBM / MALL, so that form (PF) also
//  - fetches group kg + 3's operand lines into L2 at the end of step kg
//    (one dword per 128-byte line into a scratch LDS word), so the refill
//    issued a step later hits L2;
//  - during its last steps fetches the first groups of the tile that this
//    XCD runs next in the same slot (t + CUs per XCD), so that tile's
//    prologue hits L2 as well;
//  - brings each group's block scales into the stage's tail with the refill
//    (the scales of the following group, read a step before use).
// All its direct-to-LDS loads are asm (m0 set in the same block), so the
// compiler tracks none of them and orders no LDS read behind them; a refill
// is always followed by one prefetch, so waiting for all but the newest load
// at the end of a step covers every refill.
constexpr int FB_BK = 128;                   // bytes of K per step (one scale group)
constexpr int FB_STAGE = 512 * FB_BK;        // operand bytes per stage
constexpr int FB_CP = 256 + 8;               // bf16 C-tile pitch (elements)
constexpr int FB_HALF = FB_STAGE > 128 * FB_CP * 2 ? FB_STAGE : 128 * FB_CP * 2;   // bytes per LDS array
constexpr int FB_GROUP_M = 8;
constexpr int FB_PF_MAX_GROUPS = 16;         // groups per tile up to which the PF form is used
static_assert(FB_HALF >= FB_STAGE + 512 * 4, "a stage's tail holds its 512 scale slots");

__device__ __forceinline__ int fb_sw(int row) { return (row >> 1) & 7; }
constexpr int fb_wait(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

__device__ __forceinline__ uint32_t fb_lds(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// a pointer that is the same in every lane, held in scalar registers
__device__ __forceinline__ const void* fb_sgpr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// direct-to-LDS loads of 16 / 4 bytes per lane from base + off (base the same in every
// lane): lane l's bytes land at LDS byte address lds + 16 l (4 l)
__device__ __forceinline__ void fb_dma16(const void* base, uint32_t off, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(fb_sgpr(base)),
                   "s"(lds)
                   : "memory", "m0");
}
__device__ __forceinline__ void fb_dma4(const void* base, uint32_t off, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(fb_sgpr(base)),
                   "s"(lds)
                   : "memory", "m0");
}

struct FbTile {
  int m0, n0, nbase, nend;
  const uint8_t* Wb;     // row n0 of the tile's weight matrix
  const float* wsc;      // that matrix's block scales
};

__device__ __forceinline__ FbTile fb_tile(const GemmFp8Args& g, int t, int tiles_m, int tiles_n) {
  const int span = FB_GROUP_M * tiles_n, grp = t / span, first_m = grp * FB_GROUP_M;
  const int gsz = min(tiles_m - first_m, FB_GROUP_M), r_in = t - grp * span;
  const int tn = r_in / gsz;
  const int nsp = g.W2 ? g.n_split : g.N, t1 = (nsp + 255) / 256;
  const bool second = tn >= t1;
  FbTile f;
  f.m0 = (first_m + r_in % gsz) * 256;
  f.nbase = second ? nsp : 0;                       // first row of this tile's weight matrix
  f.n0 = second ? nsp + (tn - t1) * 256 : tn * 256;
  f.nend = second ? g.N : nsp;
  const uint8_t* w = g.W;
  const float* ws = g.w_scale;
  if (second) {
    w = g.W2;
    ws = g.w2_scale;
  }
  f.Wb = w + (int64_t)(f.n0 - f.nbase) * g.K;
  f.wsc = ws;
  return f;
}

template <bool PF>
__global__ __launch_bounds__(512, 1) void gemm_fp8_big_kernel(GemmFp8Args g, int tiles_m, int tiles_n, int per_xcd,
                                                              int slots) {
  __shared__ __attribute__((aligned(16))) uint8_t s0[FB_HALF];
  __shared__ __attribute__((aligned(16))) uint8_t s1[FB_HALF];
  __shared__ __attribute__((aligned(16))) float sfirst[512];   // PF: the first group's scales
  __shared__ __attribute__((aligned(16))) uint8_t spf[256];    // PF: where L2 prefetches land
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wv >> 1, wn = wv & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int t = xcd * per_xcd + loc, ntile = tiles_m * tiles_n;
  if (loc >= per_xcd || t >= ntile) return;
  const FbTile tl = fb_tile(g, t, tiles_m, tiles_n);
  const int m0 = tl.m0, n0 = tl.n0, nbase = tl.nbase, nend = tl.nend;
  const uint8_t* Wb = tl.Wb;
  const int M = g.M, K = g.K;
  // K groups [kg0, KG) of this workgroup's split (all of them without split-K)
  const int ns = max(g.k_splits, 1), per = (K / 128 + ns - 1) / ns, split = blockIdx.y;
  const int kg0 = split * per, KG = min(K / 128, kg0 + per);
  const int nblocks = (nend - nbase + 127) / 128;
  const int wblk = min((n0 - nbase) / 128 + wn, nblocks - 1);

  // load i of wave w fills 1 KB block 8 i + w: blocks 0..31 are A rows, 32..63 W rows
  int voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (8 * i + wv) + (lane >> 3), c = (lane & 7) ^ fb_sw(r);
    if (i < 4) voff[i] = min(m0 + r, M - 1) * K + c * 16;
    else voff[i] = (min(n0 + r - 256, nend - 1) - n0) * K + c * 16;
  }

  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float srun0 = 0.f, srun1 = 0.f;

  // 32-byte fragment of row `row` (row % 32 == l32) for k half ks: logical chunks 4 ks + 2 hi, +1
  const int f = fb_sw(l32);
  int xo[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) xo[ks][e] = ((4 * ks + 2 * hi + e) ^ f) << 4;
  auto frag = [&](const uint8_t* st, int row, int ks) -> intx8 {
    const intx4 lo = *(const intx4*)(st + row * FB_BK + xo[ks][0]);
    const intx4 up = *(const intx4*)(st + row * FB_BK + xo[ks][1]);
    return (intx8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
  };
  const int ra = wm * 64 + l32, rw = 256 + wn * 128 + l32;

  // promotion: keep the sum in units of this group's scale (returns the factors for the
  // lane's two rows' sums)
  auto promote = [&](float sa0, float sa1, float sw) __attribute__((always_inline)) {
    const float n0s = sa0 * sw, n1s = sa1 * sw;
    // both quotients are formed unconditionally and selected (no branch in the wave)
    const float q0 = srun0 / n0s, q1 = srun1 / n1s;
    const float r0 = (n0s != 0.f && srun0 != 0.f) ? q0 : 1.f;
    const float r1 = (n1s != 0.f && srun1 != 0.f) ? q1 : 1.f;
    srun0 = n0s != 0.f ? n0s : srun0;
    srun1 = n1s != 0.f ? n1s : srun1;
    return make_float2(r0, r1);
  };
  // one group's MFMAs after the promotion factors r
  auto group = [&](const uint8_t* cur, float2 r) __attribute__((always_inline)) {
    const float r0 = r.x, r1 = r.y;
    // first k half: each 32x32 block is rescaled right before its MFMA, so the
    // 16 multiplies of the next block issue while the matrix core runs this
    // one; the second k half follows with no VALU work between MFMAs
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      intx8 af[2], wf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag(cur, ra + 32 * i, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = frag(cur, rw + 32 * j, ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ks == 0) {
            acc[i][j] *= i ? r1 : r0;
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // 16 VALU (the block's rescale)
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // then its MFMA
          }
          acc[i][j] = mfma32_fp8(wf[j], af[i], acc[i][j]);
        }
    }
  };

  if constexpr (!PF) {
    // (bases and sizes read from lane 0 so that the descriptors stay in scalar registers)
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)fb_sgpr(g.A), (short)0, __builtin_amdgcn_readfirstlane((int)((int64_t)M * K)), BUF_DW3);
    const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
        (void*)fb_sgpr(Wb), (short)0, __builtin_amdgcn_readfirstlane((int)((int64_t)(nend - n0) * K)), BUF_DW3);
    auto issue = [&](uint8_t* st, int kg) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < 4 ? rsA : rsW,
                                                 (__attribute__((address_space(3))) void*)(st + (8 * i + wv) * 1024),
                                                 16, voff[i], kg * FB_BK, 0, 0);
    };
    // activation scales of the lane's two output rows, the wave's weight-block scales
    const float* as0 = g.a_scale + (int64_t)min(m0 + wm * 64 + l32, M - 1) * (K / 128);
    const float* as1 = g.a_scale + (int64_t)min(m0 + wm * 64 + 32 + l32, M - 1) * (K / 128);
    const float* wsrow = tl.wsc + (int64_t)wblk * (K / 128);
    float sa0 = as0[kg0], sa1 = as1[kg0], sw = wsrow[kg0];
    auto step = [&](uint8_t* cur, int kg) {
      const float2 r = promote(sa0, sa1, sw);
      // next group's scales (clamped: the last group repeats)
      const int kn = min(kg + 1, KG - 1);
      sa0 = as0[kn];
      sa1 = as1[kn];
      sw = wsrow[kn];
      group(cur, r);
      // every wave is done with `cur` and the other stage has landed
      __builtin_amdgcn_s_waitcnt(fb_wait(0, 0));
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      issue(cur, min(kg + 2, KG - 1));
    };
    issue(s0, kg0);
    issue(s1, min(kg0 + 1, KG - 1));
    __builtin_amdgcn_s_waitcnt(fb_wait(8, 15));   // group 0 has landed
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    int kg = kg0;
    for (; kg + 1 < KG; kg += 2) {
      step(s0, kg);
      step(s1, kg + 1);
    }
    if (kg < KG) step(s0, kg);
  } else {
    // the tile this XCD's slot runs next (same split)
    const int ts = t + slots;
    const bool has_succ = loc + slots < per_xcd && ts < ntile;
    const FbTile sx = has_succ ? fb_tile(g, ts, tiles_m, tiles_n) : tl;
    // block scales of a group: waves 0-3 fetch the 256 rows' activation scales (lane 2 j + e
    // takes row 64 wv + j + 32 e, so a lane's two rows sit side by side), waves 4-7 the tile's
    // two weight blocks' (lanes 0 and 1 of wave 4 are the ones read)
    const float* sbase = g.a_scale;
    if (wv >= 4) sbase = tl.wsc + 0;
    const uint32_t soff = (uint32_t)((wv < 4 ? min(m0 + 64 * wv + (lane >> 1) + 32 * (lane & 1), M - 1)
                                             : min((n0 - nbase) / 128 + (lane & 1), nblocks - 1)) *
                                     (K / 128) * 4);
    // L2 prefetch: this thread's row (A for waves 0-3, weights for 4-7) of this tile and of the next
    const uint8_t* pb1 = g.A;
    const uint8_t* pb2 = g.A;
    if (wv >= 4) {
      pb1 = Wb + 0;
      pb2 = sx.Wb + 0;
    }
    const uint32_t pfo = (uint32_t)((wv < 4 ? min(m0 + tid, M - 1) : min(n0 + tid - 256, nend - 1) - n0) * K);
    const uint32_t pfo2 =
        (uint32_t)((wv < 4 ? min(sx.m0 + tid, M - 1) : min(sx.n0 + tid - 256, sx.nend - 1) - sx.n0) * K);
    const uint32_t lpf = fb_lds(spf);
    // group kg of this tile; past the last group, group kg - KG of the next tile (clamped)
    auto pfetch = [&](int kg) __attribute__((always_inline)) {
      if (kg < KG || !has_succ) fb_dma4(pb1 + min(kg, KG - 1) * FB_BK, pfo, lpf);
      else fb_dma4(pb2 + min(kg0 + kg - KG, KG - 1) * FB_BK, pfo2, lpf);
    };
    // a stage holds the group's 512 x 128 operand bytes, then 512 scale slots with the
    // following group's scales
    auto issue = [&](uint8_t* st, int kg) __attribute__((always_inline)) {
      const uint32_t lb = fb_lds(st);
      const uint8_t* ab = g.A + kg * FB_BK;
      const uint8_t* wb = Wb + kg * FB_BK;
#pragma unroll
      for (int i = 0; i < 8; ++i) fb_dma16(i < 4 ? ab : wb, (uint32_t)voff[i], lb + (8 * i + wv) * 1024);
      fb_dma4(sbase + min(kg + 1, KG - 1), soff, lb + FB_STAGE + 256 * wv);
    };
    struct Sc { float a0, a1, w; };
    auto read_scales = [&](const float* sc, Sc& o) __attribute__((always_inline)) {
      const float2 sa = *(const float2*)(sc + wm * 64 + 2 * l32);
      o.a0 = sa.x;
      o.a1 = sa.y;
      o.w = sc[256 + wn];
    };
    Sc scA, scB;
    auto step = [&](uint8_t* cur, const uint8_t* other, int kg, Sc& scl) __attribute__((always_inline)) {
      group(cur, promote(scl.a0, scl.a1, scl.w));
      // every wave is done with `cur`, and everything but the newest prefetch has landed
      __builtin_amdgcn_s_waitcnt(fb_wait(1, 0));
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      // `other` holds group kg + 1 and the scales of group kg + 2 (used two steps on)
      if (kg + 2 < KG) read_scales((const float*)(other + FB_STAGE), scl);
      __asm__ volatile("" ::: "memory");
      if (kg + 2 < KG) issue(cur, kg + 2);
      if (kg + 1 < KG) pfetch(kg + 3);
      __asm__ volatile("" ::: "memory");
    };
    fb_dma4(sbase + kg0, soff, fb_lds(sfirst) + 256 * wv);
    issue(s0, kg0);
    issue(s1, min(kg0 + 1, KG - 1));
    pfetch(kg0 + 2);
    __builtin_amdgcn_s_waitcnt(fb_wait(10, 15));   // group 0 and the first scales have landed
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    read_scales(sfirst, scA);
    read_scales((const float*)(s0 + FB_STAGE), scB);
    int kg = kg0;
    for (; kg + 1 < KG; kg += 2) {
      step(s0, s1, kg, scA);
      step(s1, s0, kg + 1, scB);
    }
    if (kg < KG) step(s0, s1, kg, scA);
  }
  __builtin_amdgcn_s_waitcnt(fb_wait(0, 0));
  __syncthreads();

  if (g.c_dtype == DT_F32) {
    // fp32 row-major output straight from the accumulators: a lane holds 4
    // consecutive columns of one row per result group
    float* Cf = (float*)g.C + (int64_t)split * g.split_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float sr = i ? srun1 : srun0;
      const int m = m0 + wm * 64 + i * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = n0 + wn * 128 + j * 32 + 8 * rg + 4 * hi;
          const float4 v = make_float4(acc[i][j][4 * rg] * sr, acc[i][j][4 * rg + 1] * sr,
                                       acc[i][j][4 * rg + 2] * sr, acc[i][j][4 * rg + 3] * sr);
          if (n + 4 <= nend) {
            *(float4*)(Cf + (int64_t)m * g.ldc + n) = v;
          } else {
            const float e[4] = {v.x, v.y, v.z, v.w};
            for (int k = 0; k < 4 && n + k < nend; ++k) Cf[(int64_t)m * g.ldc + n + k] = e[k];
          }
        }
    }
    return;
  }
  // epilogue: rows 0..127 of the bf16 C tile in s0, 128..255 in s1
  auto crow = [&](int row) -> uint16_t* { return (uint16_t*)(row < 128 ? s0 : s1) + (row & 127) * FB_CP; };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float sr = i ? srun1 : srun0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ml = wm * 64 + i * 32 + l32, nl = wn * 128 + j * 32 + 8 * rg + 4 * hi;
        *(uint2*)(crow(ml) + nl) = make_uint2(pack_bf16x2(acc[i][j][4 * rg] * sr, acc[i][j][4 * rg + 1] * sr),
                                              pack_bf16x2(acc[i][j][4 * rg + 2] * sr, acc[i][j][4 * rg + 3] * sr));
      }
  }
  if (g.epi == EPI_QROPE) {
    // q_b with RoPE (N = H*192): the rotary columns [192 h + 128, 192 h + 192)
    // of a head never cross a 256-column tile boundary; thread r rotates row r
    // of the staged tile for each head whose rotary columns lie in the tile,
    // with the table row of its position fetched in one batch
    float4 cs[8], sn[8];
    const int mr = min(m0 + tid, M - 1), tpos = mr % g.rope.T;
    if (tid < 256) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        cs[q] = *(const float4*)&g.rope.cos[tpos * 32 + 4 * q];
        sn[q] = *(const float4*)&g.rope.sin[tpos * 32 + 4 * q];
      }
    }
    __syncthreads();
    if (tid < 256) {
      uint16_t* r = crow(tid);
      for (int h = n0 / 192; h <= (n0 + 255) / 192; ++h) {
        const int c0 = 192 * h + 128 - n0;
        if (c0 < 0 || c0 + 64 > 256) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 x = *(const uint4*)(r + c0 + 8 * q), y = *(const uint4*)(r + c0 + 32 + 8 * q);
          uint16_t* xe = (uint16_t*)&x;
          uint16_t* ye = (uint16_t*)&y;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float4 c4 = cs[2 * q + (e >> 2)], s4 = sn[2 * q + (e >> 2)];
            const float c = (e & 3) == 0 ? c4.x : (e & 3) == 1 ? c4.y : (e & 3) == 2 ? c4.z : c4.w;
            const float sv = (e & 3) == 0 ? s4.x : (e & 3) == 1 ? s4.y : (e & 3) == 2 ? s4.z : s4.w;
            const float x1 = bf2f(xe[e]), x2 = bf2f(ye[e]);
            xe[e] = f2bf(x1 * c - x2 * sv);
            ye[e] = f2bf(x2 * c + x1 * sv);
          }
          *(uint4*)(r + c0 + 8 * q) = x;
          *(uint4*)(r + c0 + 32 + 8 * q) = y;
        }
      }
    }
  }
  __syncthreads();
  uint16_t* C = (uint16_t*)g.C;
  if (g.epi == EPI_KV_SPLIT) {
    const int h = n0 >> 8;
    for (int c = tid; c < 256 * 16; c += 512) {
      const int row = c >> 4, ch = (c & 15) * 8, m = m0 + row;
      if (m >= M) continue;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      const int64_t bh = (int64_t)bb * g.kv.H + h;
      store_nt16(C + (bh * g.kv.Tp + tt) * 128 + ch, *(const uint4*)(crow(row) + ch));
    }
    for (int c = tid; c < 256 * 16; c += 512) {
      const int row = c & 255, ch = (c >> 8) * 8, m = m0 + row;
      if (m >= M) continue;
      const uint4 v = *(const uint4*)(crow(row) + 128 + ch);
      const uint16_t* e = (const uint16_t*)&v;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      uint16_t* vt = (uint16_t*)g.kv.vt + (((int64_t)bb * g.kv.H + h) * 128 + ch) * g.kv.Tp + tt;
#pragma unroll
      for (int k = 0; k < 8; ++k) __builtin_nontemporal_store(e[k], vt + (int64_t)k * g.kv.Tp);
    }
    return;
  }
  for (int c = tid; c < 256 * 32; c += 512) {
    const int row = c >> 5, ch = (c & 31) * 8, m = m0 + row, n = n0 + ch;
    if (m >= M || n >= nend) continue;
    const uint4 v = *(const uint4*)(crow(row) + ch);
    if (n + 8 <= nend) {
      store_nt16(C + (int64_t)m * g.ldc + n, v);
    } else {
      const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < nend) C[(int64_t)m * g.ldc + n + k] = e[k];
    }
  }
}

int fb_cdiv(int a, int b) { return (a + b - 1) / b; }

// workgroups of the big kernel one XCD runs at once (one per CU): the distance from a tile to
// the one the same slot runs next
int fb_slots_per_xcd() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 32;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  const int slots = cus >= 8 ? cus / 8 : 1;
  if (dev >= 0 && dev < 64) cached[dev] = slots;
  return slots;
}
bool fp8_big_ok(const GemmFp8Args& g) {
  const int nsp = g.W2 ? g.n_split : g.N;
  return (g.c_dtype == DT_BF16 || (g.c_dtype == DT_F32 && g.epi == EPI_ROWMAJOR && (g.ldc & 3) == 0)) && g.M >= 256 && (g.N >= 256 || g.k_splits > 1) && g.K % 128 == 0 && (int64_t)g.M * g.K < (1LL << 31) &&
         (int64_t)g.N * g.K < (1LL << 31) && (!g.W2 || (nsp % 128 == 0 && nsp < g.N)) &&
         (g.epi != EPI_KV_SPLIT || g.N % 256 == 0) && (g.ldc & 7) == 0 && (((uintptr_t)g.C) & 15) == 0 &&
         (((uintptr_t)g.A | (uintptr_t)g.W | (uintptr_t)g.W2) & 15) == 0;
}

}  // namespace

bool gemm_fp8_qrope_ok(const GemmFp8Args& g) {
  return fp8_big_ok(g) && !g.W2 && g.N % 192 == 0 && g.rope.cos && g.rope.sin && g.rope.T > 0 &&
         (((uintptr_t)g.rope.cos | (uintptr_t)g.rope.sin) & 15) == 0;
}

hipError_t launch_gemm_fp8(const GemmFp8Args& g, hipStream_t s) {
  if (g.epi == EPI_QROPE && !gemm_fp8_qrope_ok(g)) return hipErrorInvalidValue;
  if (g.k_splits > 1 && (!fp8_big_ok(g) || g.c_dtype != DT_F32 || g.epi != EPI_ROWMAJOR ||
                         fb_cdiv(g.K / 128, fb_cdiv(g.K / 128, g.k_splits)) != g.k_splits ||   // no empty chunk
                         g.split_stride < (int64_t)(g.M - 1) * g.ldc + g.N))
    return hipErrorInvalidValue;
  if (fp8_big_ok(g)) {
    const int nsp = g.W2 ? g.n_split : g.N;
    const int tm = fb_cdiv(g.M, 256), tn = g.W2 ? fb_cdiv(nsp, 256) + fb_cdiv(g.N - nsp, 256) : fb_cdiv(g.N, 256);
    const int per_xcd = fb_cdiv(tm * tn, 8);
    const dim3 grid(8 * per_xcd, g.k_splits > 1 ? g.k_splits : 1);
    const int groups = fb_cdiv(g.K / 128, g.k_splits > 1 ? g.k_splits : 1);
    if (groups <= FB_PF_MAX_GROUPS)
      gemm_fp8_big_kernel<true><<<grid, 512, 0, s>>>(g, tm, tn, per_xcd, fb_slots_per_xcd());
    else
      gemm_fp8_big_kernel<false><<<grid, 512, 0, s>>>(g, tm, tn, per_xcd, 0);
    return hipGetLastError();
  }
  dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, 1);
  gemm_fp8_kernel<128, 128, 2, 2><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mla
