// bf16 GEMM on gfx950 MFMA: C = A . W^T (a bias-free Linear with [out, in]
// weights, as every MLA projection is; Kimi K2 · Output projection formula).
//
// Tiling: a 256-thread workgroup (4 waves, 64 lanes) owns a BM x BN tile of
// C and walks K in 64-wide steps. A and W tiles are staged through LDS with a
// padded 144-byte row pitch (conflict-free 16-byte reads), double-buffered
// so the next tile's global loads are in flight while MFMAs consume the
// current one. Each wave owns a (BM/WGM) x (BN/WGN) sub-tile made of 32x32
// v_mfma_f32_32x32x16_bf16 blocks with fp32 accumulators.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;

template <int BM, int BN, int WGM, int WGN, bool W_KN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * BK / 8 / 256;
  constexpr int WCH = BN * BK / 8 / 256;
  static_assert(ACH >= 1 && WCH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const uint16_t* A = (const uint16_t*)g.A + (int64_t)blockIdx.z * g.batch_a;
  const uint16_t* W = (const uint16_t*)g.W + (int64_t)blockIdx.z * g.batch_w;
  const uint16_t* W2 = (const uint16_t*)g.W2;
  const int M = g.M, N = g.N, K = g.K;

  // Per-thread chunk descriptors (16 bytes = 8 bf16 each).
  const uint16_t* a_ptr[ACH];
  int a_lds[ACH], a_k[ACH];
  bool a_ok[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
    a_ok[i] = (m0 + row) < M;
    a_ptr[i] = A + (int64_t)(a_ok[i] ? m0 + row : 0) * g.lda + col;
    a_lds[i] = row * LDK + col;
    a_k[i] = col;
  }
  const uint16_t* w_ptr[WCH];
  int w_lds[WCH], w_k[WCH];
  bool w_ok[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    int c = tid + 256 * i;
    if (!W_KN) {
      int row = c >> 3, col = (c & 7) * 8, n = n0 + row;
      w_ok[i] = n < N;
      int nn = w_ok[i] ? n : 0;
      w_ptr[i] = (nn < g.n_split ? W + (int64_t)nn * g.ldw : W2 + (int64_t)(nn - g.n_split) * g.ldw2) + col;
      w_lds[i] = row * LDK + col;
      w_k[i] = col;
    } else {
      int k = c / (BN / 8), n8 = (c % (BN / 8)) * 8;
      w_ok[i] = (n0 + n8) < N;
      w_ptr[i] = W + (int64_t)k * g.ldw + (w_ok[i] ? n0 + n8 : 0);
      w_lds[i] = n8 * LDK + k;
      w_k[i] = k;
    }
  }

  uint4 ra[ACH], rw[WCH];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      bool ok = a_ok[i] && (k0 + a_k[i]) < K;
      ra[i] = ok ? *(const uint4*)(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      bool ok = w_ok[i] && (k0 + w_k[i]) < K;
      rw[i] = ok ? *(const uint4*)(w_ptr[i] + (W_KN ? (int64_t)k0 * g.ldw : k0)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(uint4*)&sA[buf][a_lds[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      if (!W_KN) {
        *(uint4*)&sW[buf][w_lds[i]] = rw[i];
      } else {
        const uint16_t* e = (const uint16_t*)&rw[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) sW[buf][w_lds[i] + j * LDK] = e[j];
      }
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[FM], bw[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8*)&sA[cur][(wm * WM + i * 32 + lrow) * LDK + kk * 16 + lk];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bw[j] = *(const bf16x8*)&sW[cur][(wn * WN + j * 32 + lrow) * LDK + kk * 16 + lk];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bw[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column (lane % 32) and 16 rows of each 32x32 block.
  const int64_t cz = (int64_t)blockIdx.z * g.batch_c;
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
        if (g.epi == EPI_KV_SPLIT) {
          kv_split_store(g.kv, (uint16_t*)g.C, (uint16_t*)g.kv.vt, m, n, f2bf(acc[i][j][r]));
        } else if (g.c_dtype == DT_F32) {
          ((float*)g.C)[cz + (int64_t)m * g.ldc + n] = acc[i][j][r];
        } else {
          ((uint16_t*)g.C)[cz + (int64_t)m * g.ldc + n] = f2bf(acc[i][j][r]);
        }
      }
    }
}

template <int BM, int BN, int WGM, int WGN, bool KN>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch);
  gemm_bf16_kernel<BM, BN, WGM, WGN, KN><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large-shape kernel: 256x256 tile per workgroup, 4 waves of 128x128 (4x4
// blocks of 32x32, accumulators in AGPRs). K moves in 64-wide steps through a
// 2-stage LDS ring (2 x 64 KB) filled by 16-byte direct-to-LDS loads, so rows
// are whole 128-byte lines and no registers stage the data. The operand
// fragments of the next 16-wide MFMA step are read from LDS while the current
// step's 16 MFMAs run; one barrier per 64-wide step, after which that step's
// stage is refilled with the step after next. 16-byte chunks of a row are
// XOR-swizzled by (row ^ row >> 3) & 7: conflict-free operand reads with 32 or
// 64 LDS banks. Tiles are numbered so that each XCD (workgroup id % 8) works
// on a contiguous, M-grouped block of the output and its L2 serves the shared
// A/W slabs. The bf16 epilogue goes through LDS for 16-byte coalesced stores.
constexpr int GB_BM = 256, GB_BN = 256, GB_BK = 64;
constexpr int GB_STAGE = (GB_BM + GB_BN) * GB_BK;   // elements per stage (64 KB)
constexpr int GB_CP = GB_BN + 8;                   // epilogue C-tile pitch (elements)
constexpr int GB_SMEM = 2 * GB_STAGE > GB_BM * GB_CP ? 2 * GB_STAGE : GB_BM * GB_CP;
constexpr int GB_GROUP_M = 8;

__device__ __forceinline__ int gb_sw(int row) { return (row ^ (row >> 3)) & 7; }

__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(GemmArgs g, int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[GB_SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, hi = lane >> 5;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int t = xcd * per_xcd + loc, ntile = tiles_m * tiles_n;
  if (loc >= per_xcd || t >= ntile) return;
  const int span = GB_GROUP_M * tiles_n, grp = t / span, first_m = grp * GB_GROUP_M;
  const int gsz = min(tiles_m - first_m, GB_GROUP_M), r_in = t - grp * span;
  const int m0 = (first_m + r_in % gsz) * GB_BM, n0 = (r_in / gsz) * GB_BN;
  const int M = g.M, N = g.N, K = g.K, z = blockIdx.y;
  const uint16_t* A = (const uint16_t*)g.A + (int64_t)z * g.batch_a;
  const uint16_t* W = (const uint16_t*)g.W + (int64_t)z * g.batch_w;
  const uint16_t* W2 = (const uint16_t*)g.W2;

  // Direct-load slots: a stage holds A rows 0..255 then W rows 0..255, 8
  // chunks per row (4096 slots); wave w fills 1 KB blocks 16w..16w+15.
  const uint16_t* src[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = (wave * 16 + i) * 64 + lane;
    const int q = p & 2047, r = q >> 3, c = (q & 7) ^ gb_sw(r);
    if (p < 2048) {
      const int m = min(m0 + r, M - 1);
      src[i] = A + (int64_t)m * g.lda + c * 8;
    } else {
      const int n = min(n0 + r, N - 1);
      src[i] = (n < g.n_split ? W + (int64_t)n * g.ldw : W2 + (int64_t)(n - g.n_split) * g.ldw2) + c * 8;
    }
  }
  auto issue = [&](int kt) {
    uint16_t* st = smem + (kt & 1) * GB_STAGE + wave * 16 * 512;
#pragma unroll
    for (int i = 0; i < 16; ++i) __builtin_amdgcn_global_load_lds(src[i] + kt * GB_BK, st + i * 512, 16, 0, 0);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // swizzled chunk offsets of this lane's rows: the row of fragment i is
  // 128 w + 32 i + l32, whose swizzle depends on l32 and on the parity of i
  int xo[2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xo[par][kk] = ((2 * kk + hi) ^ gb_sw(32 * par + l32)) << 3;
  bf16x8 fa[2][4], fb[2][4];   // fragments of one 16-wide step, double-buffered
  auto read = [&](int kt, int kk, int buf) {
    const uint16_t* st = smem + (kt & 1) * GB_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[buf][i] = *(const bf16x8*)(st + (wm * 128 + i * 32 + l32) * GB_BK + xo[i & 1][kk]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = *(const bf16x8*)(st + GB_BM * GB_BK + (wn * 128 + j * 32 + l32) * GB_BK + xo[j & 1][kk]);
  };

  const int nk = K / GB_BK;
  issue(0);
  if (nk > 1) {
    issue(1);
    __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  read(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1;
      if (kk < 3) {
        read(kt, kk + 1, cb ^ 1);
      } else if (kt + 1 < nk) {
        // every wave holds step kt in registers and step kt+1 has landed: a
        // bare barrier (no fence, so nothing else is waited for), then stage
        // kt & 1 takes step kt+2
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (kt + 2 < nk) issue(kt + 2);
        read(kt + 1, 0, cb ^ 1);
      }
      // operands swapped (W first): a lane's accumulator holds one row of C
      // and 4 consecutive columns per group of 4 results
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fb[cb][j], fa[cb][i], acc[i][j]);
    }
  }

  // Epilogue through LDS: the bf16 C tile is staged row-major (8-byte writes
  // of 4 consecutive columns), then stored in 16-byte pieces (row-major C or
  // the k_nope part of the KV split), or as 2-byte stores running along t
  // (the transposed v part).
  __syncthreads();   // every wave is done reading the ring
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ml = wm * 128 + i * 32 + l32, nl = wn * 128 + j * 32 + 8 * rg + 4 * hi;
        *(uint2*)&smem[ml * GB_CP + nl] =
            make_uint2(pack_bf16x2(acc[i][j][4 * rg], acc[i][j][4 * rg + 1]),
                       pack_bf16x2(acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]));
      }
  __syncthreads();
  uint16_t* C = (uint16_t*)g.C + (int64_t)z * g.batch_c;
  for (int c = tid; c < GB_BM * (GB_BN / 8); c += 256) {
    const int row = c & (GB_BM - 1), ch = (c >> 8) * 8, m = m0 + row, n = n0 + ch;
    if (m >= M || n >= N) continue;
    const uint4 v = *(const uint4*)&smem[row * GB_CP + ch];
    const uint16_t* e = (const uint16_t*)&v;
    if (g.epi == EPI_KV_SPLIT) {
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T, h = n >> 8, jj = n & 255;
      const int64_t bh = (int64_t)bb * g.kv.H + h;
      if (jj < 128) {
        *(uint4*)(C + (bh * g.kv.Tp + tt) * 128 + jj) = v;
      } else {
        uint16_t* vt = (uint16_t*)g.kv.vt + (bh * 128 + (jj - 128)) * g.kv.Tp + tt;
#pragma unroll
        for (int k = 0; k < 8; ++k) vt[(int64_t)k * g.kv.Tp] = e[k];
      }
    } else if (n + 8 <= N) {
      *(uint4*)(C + (int64_t)m * g.ldc + n) = v;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < N) C[(int64_t)m * g.ldc + n + k] = e[k];
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.w_kn) return run<128, 128, 2, 2, true>(g, s);
  // bf16 output, 16-byte aligned rows (the KV split needs N % 256 == 0, true for H*256)
  const bool c_ok = g.c_dtype == DT_BF16 && (((uintptr_t)g.C) & 15) == 0 &&
                    (g.epi == EPI_KV_SPLIT ? (g.N & 255) == 0 : ((g.ldc & 7) == 0 && (g.batch_c & 7) == 0));
  const bool big = c_ok && g.M >= 256 && g.N >= 256 && g.K % GB_BK == 0 && (g.lda & 7) == 0 && (g.ldw & 7) == 0 &&
                   (g.n_split >= g.N || (g.ldw2 & 7) == 0) &&
                   (((uintptr_t)g.A | (uintptr_t)g.W | (uintptr_t)g.W2) & 15) == 0;
  if (big) {
    const int tm = (g.M + GB_BM - 1) / GB_BM, tn = (g.N + GB_BN - 1) / GB_BN;
    const int per_xcd = (tm * tn + 7) / 8;
    gemm_bf16_big_kernel<<<dim3(8 * per_xcd, g.batch), 256, 0, s>>>(g, tm, tn, per_xcd);
    return hipGetLastError();
  }
  return run<128, 128, 2, 2, false>(g, s);
}

}  // namespace mla
