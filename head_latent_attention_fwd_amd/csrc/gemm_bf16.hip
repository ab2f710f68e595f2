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
// Large-shape kernel: a BM x BN tile per 256-thread workgroup (BM = 32 WM FM,
// BN = 32 WN FN; WM x WN waves, each FM x FN blocks of 32x32 with accumulators
// in AGPRs). Shapes: 256x256 (2x2 waves of 4x4), 256x192 (2x2 of 4x3) and
// 256x224 (4x1 of 2x7); the narrower tiles make the tile count a multiple of
// the 256 CUs for N = 12288 and N = 7168.
//
// K moves in 64-wide steps through two LDS stages that are distinct LDS
// objects, so the code for each is straight-line and the compiler's waits for
// the direct-to-LDS loads never cover the other stage. A stage holds BM rows of
// A and BN rows of W, 128 bytes per row, filled by 16-byte raw-buffer loads
// straight into LDS (a per-lane byte offset fixed for the whole K loop plus a
// scalar k offset); chunks of a row are XOR-swizzled by (row >> 1) & 7, which
// spreads the 16 lanes of every 16-byte operand read over all LDS banks.
// Within a step the fragments of the next 16-wide sub-step are read between
// the MFMAs of the current one. In the last sub-step every wave waits for the
// other stage to land, one barrier retires the stage just consumed, and the
// first fragments of the other stage are read between that sub-step's MFMAs;
// the refill of the retired stage (the step two ahead) goes out in thirds
// over that sub-step and the first two of the next step. Tiles are numbered so that each
// XCD (workgroup id % 8) works on a contiguous, M-grouped block of the output
// and its L2 serves the shared A/W slabs. Output: bf16 through LDS with
// 16-byte coalesced stores (row-major or the k_nope / v^T split of kv_b), or
// fp32 split-K partials through a per-wave LDS patch.
constexpr int GB_BK = 64, GB_GROUP_M = 8;

__device__ __forceinline__ int gb_sw(int row) { return (row >> 1) & 7; }

// s_waitcnt immediate: vmcnt (6 bits, split), expcnt 7, lgkmcnt (4 bits)
constexpr int gb_wait(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

template <int WM, int WN, int FM, int FN>
struct BigTile {
  static constexpr int BM = 32 * WM * FM, BN = 32 * WN * FN;
  static constexpr int ROWS = BM + BN;
  static constexpr int LOADS = ROWS / 32;   // 16-byte loads per thread per stage
  static constexpr int STAGE = ROWS * GB_BK;   // elements
  static constexpr int CP = BN + 8;            // bf16 C-tile pitch (elements); rows 0..127 / 128..255 in stage 0 / 1
  static constexpr int FP = 32 * FN + 4;       // fp32 per-wave patch pitch (floats)
  static constexpr int HALF = (STAGE > 128 * CP ? STAGE : 128 * CP);
  static_assert(WM * WN == 4 && BM == 256 && ROWS % 32 == 0, "four waves over 256 rows");
  static_assert(2 * HALF * 2 <= 160 * 1024, "LDS budget");
  static_assert(2 * 32 * FP * 4 <= HALF * 2, "split-K patches of two waves per stage");
};

template <int WM, int WN, int FM, int FN, bool PAIRED = false>
__device__ __forceinline__ void gemm_bf16_big(const GemmArgs& g, int tiles_m, int tiles_n, int per_xcd) {
  using TL = BigTile<WM, WN, FM, FN>;
  constexpr int BM = TL::BM, BN = TL::BN, LOADS = TL::LOADS, CP = TL::CP, HALF = TL::HALF;
  __shared__ __attribute__((aligned(16))) uint16_t s0[HALF];
  __shared__ __attribute__((aligned(16))) uint16_t s1[HALF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wv / WN, wn = wv % WN, l32 = lane & 31, hi = lane >> 5;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int t = xcd * per_xcd + loc, ntile = tiles_m * tiles_n;
  if (loc >= per_xcd || t >= ntile) return;
  const int span = GB_GROUP_M * tiles_n, grp = t / span, first_m = grp * GB_GROUP_M;
  const int gsz = min(tiles_m - first_m, GB_GROUP_M), r_in = t - grp * span;
  const int m0 = (first_m + r_in % gsz) * BM, tn = r_in / gsz;
  const int M = g.M, N = g.N, K = g.K;
  const int split = g.k_splits > 1 ? (int)blockIdx.y : 0, z = g.k_splits > 1 ? 0 : (int)blockIdx.y;
  // With a second weight (rows n_split.. of the concatenated W), column tiles
  // never straddle n_split: tiles 0..t1-1 cover [0, n_split), the rest
  // [n_split, N). nend bounds the tile's region (rows past it are clamped).
  //
  // PAIRED (SwiGLU gate / up, BN = 256): tile tn produces output columns
  // [128 tn, 128 tn + 128); its W rows 0..127 are gate rows (W) and 128..255
  // the same rows of up (W2), so the epilogue holds both halves of each column.
  static_assert(!PAIRED || BN == 256, "paired tiles are 256 wide");
  const int nsp = (g.W2 && !PAIRED) ? g.n_split : N, t1 = (nsp + BN - 1) / BN;
  const bool second = !PAIRED && tn >= t1;
  const int n0 = PAIRED ? tn * 128 : second ? nsp + (tn - t1) * BN : tn * BN, nend = second ? N : nsp;
  // K chunk of this workgroup (whole K without split-K)
  const int ksteps = K / GB_BK, per = (ksteps + max(g.k_splits, 1) - 1) / max(g.k_splits, 1);
  const int kbeg = split * per * GB_BK;
  const int nk = min(per, ksteps - split * per);
  const uint16_t* A = (const uint16_t*)g.A + (int64_t)z * g.batch_a + kbeg;
  const int64_t ldw = second ? g.ldw2 : g.ldw;

  // Load slot i of wave w fills 1 KB block 4 i + w of a stage (8 rows of 8
  // chunks); blocks 0..31 are A rows, the rest W rows. Rows past M or nend
  // are clamped to the last one (loaded, never stored).
  const uint16_t* Wb = second ? (const uint16_t*)g.W2 + kbeg + (int64_t)(n0 - nsp) * g.ldw2   // row n0 of the tile
                              : (const uint16_t*)g.W + (int64_t)z * g.batch_w + kbeg + (int64_t)n0 * g.ldw;
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(((int64_t)(M - 1) * g.lda + K - kbeg) * 2), BUF_DW3);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Wb, (short)0, (int)(((int64_t)(nend - 1 - n0) * ldw + K - kbeg) * 2), BUF_DW3);
  const __amdgpu_buffer_rsrc_t rsW2 =
      PAIRED ? __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)g.W2 + kbeg + (int64_t)n0 * g.ldw2), (short)0,
                                                 (int)(((int64_t)(nend - 1 - n0) * g.ldw2 + K - kbeg) * 2), BUF_DW3)
             : rsW;
  int voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = 8 * (4 * i + wv) + (lane >> 3), c = (lane & 7) ^ gb_sw(r);
    if (i < 8) voff[i] = (int)(((int64_t)min(m0 + r, M - 1) * g.lda + c * 8) * 2);
    else if (PAIRED)   // slots 8..11: gate rows, 12..15: up rows (row r - BM - 128)
      voff[i] = (int)(((int64_t)(min(n0 + ((r - BM) & 127), nend - 1) - n0) * (i < 12 ? g.ldw : g.ldw2) + c * 8) * 2);
    else voff[i] = (int)(((int64_t)(min(n0 + r - BM, nend - 1) - n0) * ldw + c * 8) * 2);
  }
  // loads i0 <= i < i1 of step kt into stage st
  auto issue = [&](uint16_t* st, int kt, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (i < i0 || i >= i1) continue;
      auto* lds = (__attribute__((address_space(3))) void*)(st + (4 * i + wv) * 512);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(i < 8 ? rsA : (PAIRED && i >= 12 ? rsW2 : rsW), lds, 16, voff[i],
                                               kt * 128, 0, 0);
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // lane's row offsets in a stage; the swizzle depends on l32 only
  const int ra = (wm * FM * 32 + l32) * GB_BK, rw = (BM + wn * FN * 32 + l32) * GB_BK;
  int xo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) xo[kk] = ((2 * kk + hi) ^ gb_sw(l32)) << 3;
  bf16x8 fa[2][FM], fb[2][FN];   // fragments of one 16-wide sub-step, double-buffered
  auto read = [&](const uint16_t* st, int kk, int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[buf][i] = *(const bf16x8*)(st + ra + i * 32 * GB_BK + xo[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = *(const bf16x8*)(st + rw + j * 32 * GB_BK + xo[kk]);
  };
  // operands swapped (W first): a lane's accumulator holds one row of C and
  // 4 consecutive columns per group of 4 results
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fb[buf][j], fa[buf][i], acc[i][j]);
  };
  constexpr int NF = FM + FN, NMMA = FM * FN;
  // The refill of a stage goes out in thirds: the first after the barrier
  // that retires it, the other two in the first two sub-steps of the next
  // step, so the loads never arrive in one burst.
  constexpr int L1 = LOADS / 3, L2 = 2 * LOADS / 3;
  // one 64-wide step on stage `cur` (kt is the step's index); on return the
  // first fragments of the other stage are in flight to fa/fb[0]
  auto step = [&](uint16_t* cur, uint16_t* nxt, int kt) {
    const int knext = min(kt + 1, nk - 1);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      __builtin_amdgcn_s_waitcnt(gb_wait(63, 0));   // fragments of sub-step kk are in
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) issue(nxt, knext, L1, L2);
      if (kk == 1) issue(nxt, knext, L2, LOADS);
      read(cur, kk + 1, (kk + 1) & 1);
      mma(kk & 1);
      if (kk < 2) {
        constexpr int NL = L2 - L1 > LOADS - L2 ? L2 - L1 : LOADS - L2;
#pragma unroll
        for (int u = 0; u < NMMA; ++u) {
          if (u < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (u < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMMA - NF, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // every fragment of `cur` is in registers and the other stage has landed
    // (its loads are the only ones in flight): retire `cur` and start its
    // refill with the step two ahead (clamped: a repeated last step is loaded
    // and ignored)
    __builtin_amdgcn_s_waitcnt(gb_wait(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(cur, min(kt + 2, nk - 1), 0, L1);
    read(nxt, 0, 0);
    mma(1);
#pragma unroll
    for (int u = 0; u < NMMA; ++u) {
      if (u < L1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(s0, 0, 0, LOADS);
  issue(s1, min(1, nk - 1), 0, L1);
  __builtin_amdgcn_s_waitcnt(gb_wait(L1, 15));   // step 0 has landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read(s0, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(s0, s1, kt);
    step(s1, s0, kt + 1);
  }
  if (kt < nk) step(s0, s1, kt);
  // the repeated loads of the last steps land before the stages are reused
  __builtin_amdgcn_s_waitcnt(gb_wait(0, 0));
  __syncthreads();

  if (g.k_splits > 1) {
    // fp32 partial sums: each wave stages 32 rows x 32 FN columns at a time in
    // its own patch, then stores them row by row with 16-byte stores
    constexpr int FP = TL::FP, CW = FN * 8;   // lanes per row (4 floats each)
    float* P = g.part + (int64_t)split * M * N;
    float* patch = (float*)((wv >> 1) ? s1 : s0) + (wv & 1) * 32 * FP;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *(float4*)&patch[l32 * FP + j * 32 + 8 * rg + 4 * hi] =
              make_float4(acc[i][j][4 * rg], acc[i][j][4 * rg + 1], acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]);
      __builtin_amdgcn_s_waitcnt(gb_wait(63, 0));
      __builtin_amdgcn_wave_barrier();
      for (int c = lane; c < 32 * CW; c += 64) {
        const int row = c / CW, ch = (c % CW) * 4;
        const int m = m0 + wm * FM * 32 + i * 32 + row, n = n0 + wn * FN * 32 + ch;
        if (m >= M || n >= nend) continue;
        const float4 v = *(const float4*)&patch[row * FP + ch];
        float* p = P + (int64_t)m * N + n;
        if (n + 4 <= nend) {
          *(float4*)p = v;
        } else {
          const float e[4] = {v.x, v.y, v.z, v.w};
          for (int k = 0; n + k < nend; ++k) p[k] = e[k];
        }
      }
      __builtin_amdgcn_s_waitcnt(gb_wait(63, 0));
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  // Epilogue through LDS: the bf16 C tile is staged row-major (8-byte writes
  // of 4 consecutive columns; rows 0..127 in stage 0, 128..255 in stage 1),
  // then stored in 16-byte pieces.
  auto crow = [&](int row) -> uint16_t* { return (row < 128 ? s0 : s1) + (row & 127) * CP; };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      __builtin_amdgcn_sched_barrier(0);   // one block of accumulators at a time
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ml = wm * FM * 32 + i * 32 + l32, nl = wn * FN * 32 + j * 32 + 8 * rg + 4 * hi;
        *(uint2*)(crow(ml) + nl) = make_uint2(pack_bf16x2(acc[i][j][4 * rg], acc[i][j][4 * rg + 1]),
                                              pack_bf16x2(acc[i][j][4 * rg + 2], acc[i][j][4 * rg + 3]));
      }
    }
  if (BN == 192 && g.epi == EPI_QROPE) {
    // q_b with RoPE: the tile is one head, columns 128 + d and 160 + d
    // (d < 32) are the rotated pairs. Thread r rotates row r of the staged
    // tile in place; the table row of its position m % T is fetched in one
    // batch of loads while the staging completes.
    const int m = min(m0 + tid, M - 1), t = m % g.rope.T;
    float4 cs[8], sn[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      cs[q] = *(const float4*)&g.rope.cos[t * 32 + 4 * q];
      sn[q] = *(const float4*)&g.rope.sin[t * 32 + 4 * q];
    }
    __syncthreads();
    uint16_t* r = crow(tid);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 a = *(const uint4*)(r + 128 + 8 * q), b = *(const uint4*)(r + 160 + 8 * q);
      uint16_t* ae = (uint16_t*)&a;
      uint16_t* be = (uint16_t*)&b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 c4 = cs[2 * q + (e >> 2)], s4 = sn[2 * q + (e >> 2)];
        const float c = (e & 3) == 0 ? c4.x : (e & 3) == 1 ? c4.y : (e & 3) == 2 ? c4.z : c4.w;
        const float sv = (e & 3) == 0 ? s4.x : (e & 3) == 1 ? s4.y : (e & 3) == 2 ? s4.z : s4.w;
        const float x1 = bf2f(ae[e]), x2 = bf2f(be[e]);
        ae[e] = f2bf(x1 * c - x2 * sv);
        be[e] = f2bf(x2 * c + x1 * sv);
      }
      *(uint4*)(r + 128 + 8 * q) = a;
      *(uint4*)(r + 160 + 8 * q) = b;
    }
  }
  __syncthreads();
  uint16_t* C = (uint16_t*)g.C + (int64_t)z * g.batch_c;
  if (PAIRED) {
    // h[m, n0 + j] = silu(gate) * up from columns j and 128 + j of the staged tile
    for (int c = tid; c < BM * 16; c += 256) {
      const int row = c >> 4, ch = (c & 15) * 8, m = m0 + row, n = n0 + ch;
      if (m >= M || n >= nend) continue;
      const uint4 gv = *(const uint4*)(crow(row) + ch), uv = *(const uint4*)(crow(row) + 128 + ch);
      const uint16_t* ge = (const uint16_t*)&gv;
      const uint16_t* ue = (const uint16_t*)&uv;
      float h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gf = bf2f(ge[e]);
        h[e] = gf / (1.0f + __builtin_amdgcn_exp2f(-gf * 1.4426950408889634f)) * bf2f(ue[e]);
      }
      const uint4 v = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                                 pack_bf16x2(h[6], h[7]));
      if (n + 8 <= nend) {
        *(uint4*)(C + (int64_t)m * g.ldc + n) = v;
      } else {
        const uint16_t* e = (const uint16_t*)&v;
        for (int k = 0; n + k < nend; ++k) C[(int64_t)m * g.ldc + n + k] = e[k];
      }
    }
    return;
  }
  if (BN == 256 && g.epi == EPI_KV_SPLIT) {
    // the tile is one head (N % 256 == 0): columns 0..127 are k_nope, stored
    // along the row (16 lanes per row); columns 128..255 are v, stored
    // transposed with lanes running along t so each column's writes coalesce
    const int h = n0 >> 8;
    for (int c = tid; c < BM * 16; c += 256) {
      const int row = c >> 4, ch = (c & 15) * 8, m = m0 + row;
      if (m >= M) continue;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      const int64_t bh = (int64_t)bb * g.kv.H + h;
      *(uint4*)(C + (bh * g.kv.Tp + tt) * 128 + ch) = *(const uint4*)(crow(row) + ch);
    }
    for (int c = tid; c < BM * 16; c += 256) {
      const int row = c & (BM - 1), ch = (c / BM) * 8, m = m0 + row;
      if (m >= M) continue;
      const uint4 v = *(const uint4*)(crow(row) + 128 + ch);
      const uint16_t* e = (const uint16_t*)&v;
      const int bb = m / g.kv.T, tt = m - bb * g.kv.T;
      uint16_t* vt = (uint16_t*)g.kv.vt + (((int64_t)bb * g.kv.H + h) * 128 + ch) * g.kv.Tp + tt;
#pragma unroll
      for (int k = 0; k < 8; ++k) vt[(int64_t)k * g.kv.Tp] = e[k];
    }
    return;
  }
  // row-major C: BN / 8 lanes per row, 16-byte stores along the row
  for (int c = tid; c < BM * (BN / 8); c += 256) {
    const int row = c / (BN / 8), ch = (c % (BN / 8)) * 8, m = m0 + row, n = n0 + ch;
    if (m >= M || n >= nend) continue;
    const uint4 v = *(const uint4*)(crow(row) + ch);
    if (n + 8 <= nend) {
      *(uint4*)(C + (int64_t)m * g.ldc + n) = v;
    } else {
      const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < nend) C[(int64_t)m * g.ldc + n + k] = e[k];
    }
  }
}

// one kernel per tile shape (plain kernels around the templated body)
__global__ __launch_bounds__(256, 1) void gemm_bf16_big256_kernel(GemmArgs g, int tm, int tn, int per_xcd) {
  gemm_bf16_big<2, 2, 4, 4>(g, tm, tn, per_xcd);
}
__global__ __launch_bounds__(256, 1) void gemm_bf16_big224_kernel(GemmArgs g, int tm, int tn, int per_xcd) {
  gemm_bf16_big<4, 1, 2, 7>(g, tm, tn, per_xcd);
}
__global__ __launch_bounds__(256, 1) void gemm_bf16_big192_kernel(GemmArgs g, int tm, int tn, int per_xcd) {
  gemm_bf16_big<2, 2, 4, 3>(g, tm, tn, per_xcd);
}
__global__ __launch_bounds__(256, 1) void gemm_bf16_swiglu_kernel(GemmArgs g, int tm, int tn, int per_xcd) {
  gemm_bf16_big<2, 2, 4, 4, true>(g, tm, tn, per_xcd);
}

}  // namespace

namespace {
// operand shapes the big-tile kernels take
// (narrow: outputs of fewer than 256 columns too, for split-K products)
bool big_ok(const GemmArgs& g, bool narrow = false) {
  // raw-buffer loads address each operand with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 31;
  const int nsp = g.W2 ? g.n_split : g.N;
  const bool fits = ((int64_t)(g.M - 1) * g.lda + g.K) * 2 < lim && ((int64_t)(nsp - 1) * g.ldw + g.K) * 2 < lim &&
                    (!g.W2 || (((int64_t)(g.N - nsp - 1) * g.ldw2 + g.K) * 2 < lim && (nsp & 7) == 0 && nsp < g.N &&
                               (g.ldw2 & 7) == 0 && ((uintptr_t)g.W2 & 15) == 0));
  return !g.w_kn && g.M >= 256 && (g.N >= 256 || (narrow && g.N >= 8)) && g.K % GB_BK == 0 && (g.lda & 7) == 0 && (g.ldw & 7) == 0 && fits &&
         (((uintptr_t)g.A | (uintptr_t)g.W) & 15) == 0;
}
int cdiv(int a, int b) { return (a + b - 1) / b; }
int big_tiles_n(const GemmArgs& g, int bn) {
  return g.W2 ? cdiv(g.n_split, bn) + cdiv(g.N - g.n_split, bn) : cdiv(g.N, bn);
}
// tile width: the widest of 256 / 224 / 192 whose tile count fills whole rounds
// of 256 CUs best (the KV split and split-K use 256)
int big_bn(const GemmArgs& g) {
  if (g.epi == EPI_KV_SPLIT || g.k_splits > 1) return 256;
  const int tm = cdiv(g.M, 256);
  int best = 256;
  double best_eff = 0;
  for (int bn : {256, 224, 192}) {
    const int tiles = tm * big_tiles_n(g, bn) * g.batch;
    const double eff = (double)tiles / (cdiv(tiles, 256) * 256.0) * ((double)g.N / (big_tiles_n(g, bn) * bn));
    if (eff > best_eff + 1e-9) { best_eff = eff; best = bn; }
  }
  return best;
}
hipError_t run_big(const GemmArgs& g, int bn, int ny, hipStream_t s) {
  const int tm = cdiv(g.M, 256), tn = big_tiles_n(g, bn);
  const int per_xcd = cdiv(tm * tn, 8);
  const dim3 grid(8 * per_xcd, ny);
  if (bn == 224) gemm_bf16_big224_kernel<<<grid, 256, 0, s>>>(g, tm, tn, per_xcd);
  else if (bn == 192) gemm_bf16_big192_kernel<<<grid, 256, 0, s>>>(g, tm, tn, per_xcd);
  else gemm_bf16_big256_kernel<<<grid, 256, 0, s>>>(g, tm, tn, per_xcd);
  return hipGetLastError();
}

// Split-K plan for outputs with too few tiles for the chip: the tile width
// and chunk count whose workgroups fill the most of one round of 256 CUs
// (counting padded columns as waste), at least 8 steps of 64 per chunk.
struct SplitPlan { int bn, splits; };
SplitPlan split_plan(const GemmArgs& g) {
  SplitPlan best{256, 1};
  if (!big_ok(g, true) || g.batch != 1 || (g.N & 3) != 0 || g.epi == EPI_KV_SPLIT) return best;
  const int tm = cdiv(g.M, 256), ksteps = g.K / GB_BK;
  double best_eff = 0;
  for (int bn : {256, 224, 192}) {
    const int tiles = tm * big_tiles_n(g, bn);
    if (tiles >= 128) continue;
    int splits = 256 / tiles;
    if (splits > ksteps / 8) splits = ksteps / 8;
    if (splits < 2) continue;
    splits = cdiv(ksteps, cdiv(ksteps, splits));   // chunks actually made
    const double eff = (double)tiles * splits / 256.0 * ((double)g.N / (big_tiles_n(g, bn) * bn));
    if (eff > best_eff + 1e-9) { best_eff = eff; best = {bn, splits}; }
  }
  return best;
}
}  // namespace

int gemm_bf16_splits(const GemmArgs& g) { return split_plan(g).splits; }

double gemm_bf16_cost(const GemmArgs& g, bool split) {
  if (split) {
    const SplitPlan p = split_plan(g);
    const int tiles = cdiv(g.M, 256) * big_tiles_n(g, p.bn) * p.splits;
    return (double)cdiv(tiles, 256) * p.bn / 256.0 / p.splits;
  }
  const int bn = big_bn(g), tiles = cdiv(g.M, 256) * big_tiles_n(g, bn) * g.batch;
  return (double)cdiv(tiles, 256) * bn / 256.0;
}

bool gemm_bf16_qrope_ok(const GemmArgs& g) {
  return big_ok(g) && !g.W2 && g.batch == 1 && g.k_splits <= 1 && g.c_dtype == DT_BF16 && g.N % 192 == 0 &&
         (g.ldc & 7) == 0 && (((uintptr_t)g.C) & 15) == 0 && g.rope.cos && g.rope.sin && g.rope.T > 0 &&
         (((uintptr_t)g.rope.cos | (uintptr_t)g.rope.sin) & 15) == 0;
}

bool gemm_bf16_swiglu_ok(const GemmArgs& g) {
  GemmArgs h = g;
  h.W2 = nullptr;   // the pairing replaces the stacked-weight split
  return big_ok(h) && g.W2 && g.batch == 1 && g.k_splits <= 1 && g.c_dtype == DT_BF16 && g.N % 128 == 0 &&
         (g.ldw2 & 7) == 0 && (((uintptr_t)g.W2) & 15) == 0 &&
         ((int64_t)(g.N - 1) * g.ldw2 + g.K) * 2 < ((int64_t)1 << 31) && (g.ldc & 7) == 0 &&
         (((uintptr_t)g.C) & 15) == 0;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.epi == EPI_QROPE) return gemm_bf16_qrope_ok(g) ? run_big(g, 192, 1, s) : hipErrorInvalidValue;
  if (g.epi == EPI_SWIGLU) {
    if (!gemm_bf16_swiglu_ok(g)) return hipErrorInvalidValue;
    const int tm = cdiv(g.M, 256), tn = g.N / 128, per_xcd = cdiv(tm * tn, 8);
    gemm_bf16_swiglu_kernel<<<8 * per_xcd, 256, 0, s>>>(g, tm, tn, per_xcd);
    return hipGetLastError();
  }
  if (g.w_kn) return run<128, 128, 2, 2, true>(g, s);
  if (g.k_splits > 1) {   // the caller sized part[] from gemm_bf16_splits
    if (!big_ok(g, true) || g.batch != 1 || !g.part || g.k_splits != gemm_bf16_splits(g)) return hipErrorInvalidValue;
    return run_big(g, split_plan(g).bn, g.k_splits, s);
  }
  // bf16 output, 16-byte aligned rows (the KV split needs N % 256 == 0, true for H*256)
  const bool c_ok = g.c_dtype == DT_BF16 && (((uintptr_t)g.C) & 15) == 0 &&
                    (g.epi == EPI_KV_SPLIT ? (g.N & 255) == 0 : ((g.ldc & 7) == 0 && (g.batch_c & 7) == 0));
  if (c_ok && big_ok(g)) {
    return run_big(g, big_bn(g), g.batch, s);
  }
  return run<128, 128, 2, 2, false>(g, s);
}

}  // namespace mla
