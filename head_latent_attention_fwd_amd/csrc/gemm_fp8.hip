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

}  // namespace

hipError_t launch_gemm_fp8(const GemmFp8Args& g, hipStream_t s) {
  dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, 1);
  gemm_fp8_kernel<128, 128, 2, 2><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mla
