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
// blocks of 32x32, accumulators in AGPRs). K moves in 32-wide steps through a
// 4-stage LDS ring (4 x 32 KB) filled by 16-byte direct-to-LDS loads; a
// step's loads are issued while the three steps before it are consumed, so
// the L2/HBM latency hides behind ~3000 cycles of math. The operand fragments of the
// next 16-wide MFMA step are read from LDS while the current step's 16 MFMAs
// run; one barrier per 32-wide step, after which the stage just consumed is
// refilled with the step four ahead. Rows are 64 bytes (4 chunks of 16 B),
// XOR-swizzled by ((row >> 1) ^ (row >> 3)) & 3: conflict-free operand reads
// with 32 or 64 LDS banks. Tiles are numbered so that each XCD (workgroup id
// % 8) works on a contiguous, M-grouped block of the output and its L2 serves
// the shared A/W slabs. The bf16 epilogue goes through LDS for 16-byte
// coalesced stores.
constexpr int GB_BM = 256, GB_BN = 256, GB_BK = 32, GB_NST = 4;
constexpr int GB_STAGE = (GB_BM + GB_BN) * GB_BK;   // elements per stage (32 KB)
constexpr int GB_LOADS = GB_STAGE / 8 / 256;        // 16-byte loads per thread per stage
constexpr int GB_CP = GB_BN + 8;                    // epilogue C-tile pitch (elements)
constexpr int GB_SMEM = GB_NST * GB_STAGE > GB_BM * GB_CP ? GB_NST * GB_STAGE : GB_BM * GB_CP;
constexpr int GB_GROUP_M = 8;

__device__ __forceinline__ int gb_sw(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// s_waitcnt vmcnt(n * GB_LOADS): stages still allowed in flight
__device__ __forceinline__ void gb_wait_stages(int n) {
  if (n >= 3) __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (n == 2) __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n == 1) __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

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
  const int M = g.M, N = g.N, K = g.K;
  const int split = g.k_splits > 1 ? (int)blockIdx.y : 0, z = g.k_splits > 1 ? 0 : (int)blockIdx.y;
  // K chunk of this workgroup (whole K without split-K)
  const int ksteps = K / GB_BK, per = (ksteps + max(g.k_splits, 1) - 1) / max(g.k_splits, 1);
  const int kbeg = split * per * GB_BK;
  const uint16_t* A = (const uint16_t*)g.A + (int64_t)z * g.batch_a + kbeg;
  const uint16_t* W = (const uint16_t*)g.W + (int64_t)z * g.batch_w + kbeg;
  const uint16_t* W2 = g.W2 ? (const uint16_t*)g.W2 + kbeg : nullptr;

  // Direct-load slots: a stage holds A rows 0..255 then W rows 0..255, 4
  // chunks per row (2048 slots); wave w fills 1 KB blocks 8w..8w+7.
  const uint16_t* src[GB_LOADS];
#pragma unroll
  for (int i = 0; i < GB_LOADS; ++i) {
    const int p = (wave * GB_LOADS + i) * 64 + lane;
    const int q = p & 1023, r = q >> 2, c = (q & 3) ^ gb_sw(r);
    if (p < 1024) {
      const int m = min(m0 + r, M - 1);
      src[i] = A + (int64_t)m * g.lda + c * 8;
    } else {
      const int n = min(n0 + r, N - 1);
      src[i] = (n < g.n_split ? W + (int64_t)n * g.ldw : W2 + (int64_t)(n - g.n_split) * g.ldw2) + c * 8;
    }
  }
  auto issue = [&](int kt) {
    uint16_t* st = smem + (kt % GB_NST) * GB_STAGE + wave * GB_LOADS * 512;
#pragma unroll
    for (int i = 0; i < GB_LOADS; ++i)
      __builtin_amdgcn_global_load_lds(src[i] + kt * GB_BK, st + i * 512, 16, 0, 0);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // swizzled chunk offset of this lane's rows (the swizzle depends on l32 only)
  int xo[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) xo[kk] = ((2 * kk + hi) ^ gb_sw(l32)) << 3;
  bf16x8 fa[2][4], fb[2][4];   // fragments of one 16-wide step, double-buffered
  auto read = [&](int kt, int kk, int buf) {
    const uint16_t* st = smem + (kt % GB_NST) * GB_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[buf][i] = *(const bf16x8*)(st + (wm * 128 + i * 32 + l32) * GB_BK + xo[kk]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[buf][j] = *(const bf16x8*)(st + GB_BM * GB_BK + (wn * 128 + j * 32 + l32) * GB_BK + xo[kk]);
  };

  const int nk = min(per, ksteps - split * per);
  for (int s = 0; s < GB_NST; ++s)
    if (s < nk) issue(s);
  gb_wait_stages(min(nk, GB_NST) - 1);   // step 0 has landed
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  read(0, 0, 0);
  // operands swapped (W first): a lane's accumulator holds one row of C and
  // 4 consecutive columns per group of 4 results
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fb[buf][j], fa[buf][i], acc[i][j]);
  };
  // Step kt: the second half of its fragments is read during the first
  // half's MFMAs; then every wave holds step kt in registers and step kt+1
  // has landed (kt+2, kt+3 may be in flight), so after a bare barrier the
  // stage of step kt takes step kt+4. The steady-state loop has no branch
  // inside, which keeps the compiler's own LDS waits tight.
  // sched_barrier(0) keeps the compiler from moving the reads behind the MFMAs
  // they are meant to overlap.
  int kt = 0;
  for (; kt + GB_NST < nk; ++kt) {
    // the first-half fragments were read a whole MFMA group ago: a builtin
    // lgkmcnt(0) here costs nothing and tells the compiler they are in
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    read(kt, 1, 1);
    mma(0);
    // one LDS read between every two MFMAs
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // s_waitcnt vmcnt(16) lgkmcnt(0) as a builtin, so the compiler's own wait
    // accounting knows the reads of this step are complete
    __builtin_amdgcn_s_waitcnt(0x4070);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + GB_NST);
    read(kt + 1, 0, 0);
    mma(1);
    // MFMAs interleaved with the refill loads and the next step's LDS reads
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; kt < nk; ++kt) {   // the last steps: nothing left to issue
    read(kt, 1, 1);
    mma(0);
    if (kt + 1 < nk) {
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      gb_wait_stages(min(nk - 2 - kt, GB_NST - 2));
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      read(kt + 1, 0, 0);
    }
    mma(1);
  }

  if (g.k_splits > 1) {
    // fp32 partial sums through LDS, one 128-row half of the tile at a time
    // (the waves with wm == half stage it), then 64 lanes per row store 1 KB
    constexpr int FP = GB_BN + 4;   // fp32 pitch
    float* P = g.part + (int64_t)split * M * N;
    float* sf = (float*)smem;
    for (int half = 0; half < 2; ++half) {
      __syncthreads();   // the ring (or the previous half) is no longer read
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
              *(float4*)&sf[(i * 32 + l32) * FP + wn * 128 + j * 32 + 8 * rg + 4 * hi] =
                  make_float4(acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]);
      }
      __syncthreads();
      for (int c = tid; c < 128 * (GB_BN / 4); c += 256) {
        const int row = c >> 6, ch = (c & 63) * 4, m = m0 + half * 128 + row, n = n0 + ch;
        if (m >= M || n >= N) continue;
        const float4 v = *(const float4*)&sf[row * FP + ch];
        float* p = P + (int64_t)m * N + n;
        if (n + 4 <= N) {
          *(float4*)p = v;
        } else {
          const float e[4] = {v.x, v.y, v.z, v.w};
          for (int k = 0; n + k < N; ++k) p[k] = e[k];
        }
      }
    }
    return;
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
  if (g.epi == EPI_KV_SPLIT) {
    // the tile is one head (N % 256 == 0): columns 0..127 are k_nope, stored
    // along the row (16 lanes per row); columns 128..255 are v, stored
    // transposed with lanes running along t so each column's writes coalesce
    const int h = n0 >> 8;
    for (int c = tid; c < GB_BM * 16; c += 256) {
      const int row = c >> 4, ch = (c & 15) * 8, m = m0 + row;
      if (m >= M) continue;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      const int64_t bh = (int64_t)bb * g.kv.H + h;
      *(uint4*)(C + (bh * g.kv.Tp + tt) * 128 + ch) = *(const uint4*)&smem[row * GB_CP + ch];
    }
    for (int c = tid; c < GB_BM * 16; c += 256) {
      const int row = c & (GB_BM - 1), ch = (c >> 8) * 8, m = m0 + row;
      if (m >= M) continue;
      const uint4 v = *(const uint4*)&smem[row * GB_CP + 128 + ch];
      const uint16_t* e = (const uint16_t*)&v;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      uint16_t* vt = (uint16_t*)g.kv.vt + (((int64_t)bb * g.kv.H + h) * 128 + ch) * g.kv.Tp + tt;
#pragma unroll
      for (int k = 0; k < 8; ++k) vt[(int64_t)k * g.kv.Tp] = e[k];
    }
    return;
  }
  // row-major C: 32 lanes per row, 16-byte stores along the row
  for (int c = tid; c < GB_BM * (GB_BN / 8); c += 256) {
    const int row = c >> 5, ch = (c & 31) * 8, m = m0 + row, n = n0 + ch;
    if (m >= M || n >= N) continue;
    const uint4 v = *(const uint4*)&smem[row * GB_CP + ch];
    if (n + 8 <= N) {
      *(uint4*)(C + (int64_t)m * g.ldc + n) = v;
    } else {
      const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < N) C[(int64_t)m * g.ldc + n + k] = e[k];
    }
  }
}

}  // namespace

namespace {
// operand shapes the big-tile kernel takes
bool big_ok(const GemmArgs& g) {
  return !g.w_kn && g.M >= 256 && g.N >= 256 && g.K % GB_BK == 0 && (g.lda & 7) == 0 && (g.ldw & 7) == 0 &&
         (g.n_split >= g.N || (g.ldw2 & 7) == 0) && (((uintptr_t)g.A | (uintptr_t)g.W | (uintptr_t)g.W2) & 15) == 0;
}
}  // namespace

int gemm_bf16_splits(const GemmArgs& g) {
  if (!big_ok(g) || g.batch != 1 || (g.N & 3) != 0) return 1;
  const int tiles = ((g.M + GB_BM - 1) / GB_BM) * ((g.N + GB_BN - 1) / GB_BN);
  if (tiles >= 128) return 1;
  int splits = 256 / tiles;
  const int ksteps = g.K / GB_BK;
  if (splits > ksteps / 16) splits = ksteps / 16;   // at least 16 steps of 32 per chunk
  if (splits < 2) return 1;
  const int per = (ksteps + splits - 1) / splits;
  return (ksteps + per - 1) / per;   // chunks actually made
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.w_kn) return run<128, 128, 2, 2, true>(g, s);
  const int tm = (g.M + GB_BM - 1) / GB_BM, tn = (g.N + GB_BN - 1) / GB_BN;
  const int per_xcd = (tm * tn + 7) / 8;
  if (g.k_splits > 1) {   // the caller sized part[] from gemm_bf16_splits
    if (!big_ok(g) || g.batch != 1 || !g.part || g.k_splits != gemm_bf16_splits(g)) return hipErrorInvalidValue;
    gemm_bf16_big_kernel<<<dim3(8 * per_xcd, g.k_splits), 256, 0, s>>>(g, tm, tn, per_xcd);
    return hipGetLastError();
  }
  // bf16 output, 16-byte aligned rows (the KV split needs N % 256 == 0, true for H*256)
  const bool c_ok = g.c_dtype == DT_BF16 && (((uintptr_t)g.C) & 15) == 0 &&
                    (g.epi == EPI_KV_SPLIT ? (g.N & 255) == 0 : ((g.ldc & 7) == 0 && (g.batch_c & 7) == 0));
  if (c_ok && big_ok(g)) {
    gemm_bf16_big_kernel<<<dim3(8 * per_xcd, g.batch), 256, 0, s>>>(g, tm, tn, per_xcd);
    return hipGetLastError();
  }
  return run<128, 128, 2, 2, false>(g, s);
}

}  // namespace mla
