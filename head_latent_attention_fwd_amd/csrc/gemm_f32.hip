// fp32 GEMM C = A . W^T for the fp32 path (small shapes; plain FMA on the
// vector ALUs, 64x64 tiles through LDS, 4x4 outputs per thread).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int TB = 64, TK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float sA[TK][TB + 4];
  __shared__ float sW[TK][TB + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const float* A = (const float*)g.A + (int64_t)blockIdx.z * g.batch_a;
  const float* W = (const float*)g.W + (int64_t)blockIdx.z * g.batch_w;
  const float* W2 = (const float*)g.W2;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
    for (int e = tid; e < TB * TK; e += 256) {
      int r = e / TK, k = e % TK;
      int m = m0 + r, n = n0 + r, kk = k0 + k;
      sA[k][r] = (m < g.M && kk < g.K) ? A[(int64_t)m * g.lda + kk] : 0.f;
      float wv = 0.f;
      if (n < g.N && kk < g.K) {
        if (g.w_kn) wv = W[(int64_t)kk * g.ldw + n];
        else wv = n < g.n_split ? W[(int64_t)n * g.ldw + kk] : W2[(int64_t)(n - g.n_split) * g.ldw2 + kk];
      }
      sW[k][r] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[k][tm + i]; b[i] = sW[k][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = (float*)g.C + (int64_t)blockIdx.z * g.batch_c;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + tm + i, n = n0 + tn + j;
      if (m >= g.M || n >= g.N) continue;
      if (g.epi == EPI_KV_SPLIT) kv_split_store(g.kv, (float*)g.C, (float*)g.kv.vt, m, n, acc[i][j]);
      else C[(int64_t)m * g.ldc + n] = acc[i][j];
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  dim3 grid((g.N + TB - 1) / TB, (g.M + TB - 1) / TB, g.batch);
  gemm_f32_kernel<<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mla
