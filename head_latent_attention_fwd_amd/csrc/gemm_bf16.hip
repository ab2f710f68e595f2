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

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.w_kn) return run<128, 128, 2, 2, true>(g, s);
  return run<128, 128, 2, 2, false>(g, s);
}

}  // namespace mla
