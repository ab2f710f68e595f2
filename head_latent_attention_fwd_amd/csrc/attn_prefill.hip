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
// With a non-empty cache the T queries sit at positions P..P+T-1 and attend
// keys 0..P+T-1 (the P cached keys come first in kn / vt / kpe); P = 0 is the
// plain prefill.
//
// Work split: one 256-thread workgroup per (two 128-query tiles, head,
// sequence): tiles nq - 1 - z and z of the pair, so all workgroups carry the
// same causal work; the pairs of an XCD are walked one after another so their
// keys and values stay in its L2; wave w owns queries [32w, 32w+32) of a tile.
// Scores are formed transposed, S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16 so
// a lane holds 32 keys of one query: the running max needs one exchange
// (lane ^ 32) and the running sum stays lane-local; the bf16 probabilities are
// the B operand of O^T = V^T . P^T. Q stays in registers.
//
// Tiles move HBM -> LDS with gfx950's 16-byte direct-to-LDS loads into a
// two-stage ring (one barrier per tile; the next tile's loads fly while the
// current tile is consumed), 40 KB per stage, two workgroups per CU. The next
// tile's ten loads per thread are issued one per two score MFMAs rather than
// ahead of them: a wave issues in order, and a burst of loads held its first
// MFMA back while the texture unit took in the workgroup's 40 KB. The tile
// loop is unrolled over the two stages so every LDS address is a per-lane
// base plus an immediate. Within a
// 16-key block the K rows are stored with bits 2 and 3 of the key index
// swapped: the 32x32 MFMA output then gives each lane 8 consecutive keys per
// 16-key step, so the matching V^T operand is one 16-byte LDS read. 16-byte
// chunks are XOR-swizzled by row in every region (conflict-free reads with 32
// or 64 LDS banks).
//
// Softmax: a query's running max is fixed at its first live keys and later
// keys add exp2(z - m) unrescaled (fp32 holds any z - m below 2^7; the bf16
// probabilities have the same exponent range), so O is never rescaled. The
// row sum adds the bf16-rounded probabilities (two per v_dot2 against ones),
// the same weights the value product uses. If the
// sum of a query then leaves [0, 2^64) (a logit jump of more than ~44 nats)
// the workgroup redoes its tile in two passes of the same loop: exact maxima
// first, then the accumulation against them.
// Masks: per 32-key block a lane builds one 32-bit word of the keys live for
// its query (selection bits, causal limit, sequence end); tiles wholly inside
// every query's causal range without a selection skip it. Every branch
// condition of the tile loop is wave-uniform.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BQ = 128;                   // queries per workgroup
constexpr int BKV = 64;                   // keys per tile
// one LDS stage (bf16 elements): k_nope [64][128] | k_pe [64][64] | v^T [128][64]
constexpr int ST_KN = 0, ST_KPE = 64 * 128, ST_VT = ST_KPE + 64 * 64, STAGE = ST_VT + 128 * 64;
constexpr int LOADS = STAGE * 2 / 16 / 256;  // 16-byte direct loads per thread per tile (10)
constexpr float LSUM_MAX = 18446744073709551616.0f;   // 2^64: a query sum beyond this ran past its fixed max

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// chunk swizzle of 128-byte rows, conflict-free for 32 or 64 LDS banks
__device__ __forceinline__ int sw8(int r) { return (r ^ (r >> 3)) & 7; }

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];   // 80 KB: two workgroups per CU

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int T = a.T, Tp = a.Tp, H = a.H, P = a.P, Tk = P + T;
  // Work order: workgroup id % 8 is the XCD; each XCD takes whole (sequence,
  // head) pairs one after another, and a workgroup takes the query tiles
  // nq - 1 - z and z of its pair (zigzag), so every workgroup has the same
  // causal work and the keys and values of the pairs in flight on an XCD stay
  // in its L2 (the second tile re-reads a prefix the first one just streamed).
  const int nq = (T + BQ - 1) / BQ, nz = (nq + 1) / 2;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int pair = (loc / nz) * 8 + xcd, z = loc % nz;
  if (pair >= a.B * H) return;
  const int h = pair % H, b = pair / H;
  const int64_t bh = (int64_t)b * H + h;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  for (int zz = 0; zz < 2; ++zz) {
  const int qt = zz ? z : nq - 1 - z;
  if (zz && qt == nq - 1 - z) break;   // odd tile count: the middle tile is alone
  const int q0 = qt * BQ, qw = q0 + wv * 32;   // wave-uniform
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

  // Direct-load slots: load i of wave w fills 1 KB block 4i + w of a stage;
  // lane l lands in 16-byte slot p = 64 (4i + w) + l. Blocks 0..15 are k_nope,
  // 16..23 k_pe and 24..39 v^T, so the region of load i is fixed by i and each
  // load reads one raw buffer: a per-lane byte offset within the tile (fixed
  // over tiles) plus a scalar tile offset.
  const __amdgpu_buffer_rsrc_t rs_kn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.kn + bh * Tp * 128), (short)0, Tp * 128 * 2, BUF_DW3);
  const __amdgpu_buffer_rsrc_t rs_kpe = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.kpe + (int64_t)b * Tp * 64), (short)0, Tp * 64 * 2, BUF_DW3);
  const __amdgpu_buffer_rsrc_t rs_vt = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)a.vt + bh * 128 * Tp), (short)0, 128 * Tp * 2, BUF_DW3);
  int voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = (4 * i + wv) * 64 + lane;
    if (i < 4) {                                // k_nope: row rho, chunk' = chunk ^ (rho & 15)
      const int rho = p >> 4, c = (p & 15) ^ (rho & 15);
      voff[i] = (swap23(rho) * 128 + c * 8) * 2;
    } else if (i < 6) {                         // k_pe
      const int q = p - ST_KPE / 8, rho = q >> 3, c = (q & 7) ^ sw8(rho);
      voff[i] = (swap23(rho) * 64 + c * 8) * 2;
    } else {                                    // v^T: row dv, 8-key chunk
      const int q = p - ST_VT / 8, dv = q >> 3, c = (q & 7) ^ sw8(dv);
      voff[i] = (dv * Tp + c * 8) * 2;
    }
  }
  auto issue_one = [&](int stage, int k0, int i) {
    auto* lds = (__attribute__((address_space(3))) void*)(smem + stage * STAGE + (4 * i + wv) * 512);
    if (i < 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kn, lds, 16, voff[i], k0 * 256, 0, 0);
    else if (i < 6) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kpe, lds, 16, voff[i], k0 * 128, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_vt, lds, 16, voff[i], k0 * 2, 0, 0);
  };
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) issue_one(stage, k0, i);
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
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;
  const int W = (Tk + 31) >> 5;
  const bool has_mask = a.mask != nullptr;   // wave-uniform (mrow is a per-lane row pointer)
  const uint32_t* mrow = has_mask ? a.mask + ((int64_t)b * T + (q_ok ? qi : 0)) * W : nullptr;
  // absolute position of this lane's query
  const int pi = P + qi;

  const int kv_end = min(Tk, P + q0 + BQ);
  const int ntiles = (kv_end + BKV - 1) / BKV;
  // selection words of a tile (two 32-key words per query row), fetched one tile
  // ahead and before the tile refill so that waiting for them never waits for it
  auto mask_words = [&](int kt, uint32_t& w0, uint32_t& w1) {
    w0 = w1 = 0xFFFFFFFFu;
    if (has_mask && kt < ntiles) {
      const int wi = (kt * BKV) >> 5;
      w0 = mrow[wi];
      w1 = wi + 1 < W ? mrow[wi + 1] : 0u;
    }
  };
  // keys j of the 32-key block starting at key kb0 that are live for this
  // lane's query, shifted so that bit 16 (r / 8) + r % 8 is the key of result
  // slot r (lane half hi holds keys 16 (r / 8) + 8 hi + r % 8)
  auto live_word = [&](uint32_t sel, int kb0) {
    const int lim = min(pi, Tk - 1) - kb0;   // keys j <= lim exist and are causal
    const uint32_t lm = lim >= 31 ? 0xFFFFFFFFu : lim < 0 ? 0u : ((2u << lim) - 1u);
    return (sel & lm) >> (8 * hi);
  };

  // mode 0: accumulate with each query's max fixed at its first live keys;
  // mode 1 (after an overflow anywhere in the workgroup): exact maxima only;
  // mode 2: accumulate against those maxima. One copy of the loop serves all
  // three (the mode is workgroup-uniform).
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  for (int mode = 0;;) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][r] = 0.f;
    // the sum runs over the bf16 probabilities that enter the value product
    // (two partial sums: shorter dependency chains)
    float l0 = 0.f, l1 = 0.f;
    uint32_t nw0, nw1;
    mask_words(0, nw0, nw1);
    issue(0, 0);
    // one tile; the stage is a compile-time constant so that every LDS address
    // is a per-lane base plus an immediate offset
    auto tile = [&](int kt, auto stage) {
      constexpr int cur = decltype(stage)::value;
      const int k0 = kt * BKV;
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const uint32_t mw0 = nw0, mw1 = nw1;
      mask_words(kt + 1, nw0, nw1);
      const bool more = kt + 1 < ntiles;   // wave-uniform
      // No early exit: a tile wholly after this wave's queries (k0 > pw) goes
      // through the masked path with every key dead, so O is updated on every
      // path and the compiler keeps it in place.
      const uint16_t* sb = smem + cur * STAGE;
      floatx16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      // step u = (kk, kb) = (u / 2, u % 2); K fragments read three steps ahead
      auto kfrag = [&](int u) {
        const int kk = u >> 1, kb = u & 1, rho = kb * 32 + l32;
        const int off = kk < 8 ? ST_KN + rho * 128 + xk[kk] : ST_KPE + rho * 64 + xp[kb][kk - 8];
        return *(const bf16x8*)(sb + off);
      };
      bf16x8 kf[24];   // one value per unrolled step (no register copies)
      kf[0] = kfrag(0);
      kf[1] = kfrag(1);
      kf[2] = kfrag(2);
#pragma unroll
      for (int u = 0; u < 24; ++u) {
        if (u + 3 < 24) kf[u + 3] = kfrag(u + 3);
        // the next tile's loads go out one per two MFMAs instead of ahead of them
        if ((u & 1) == 0 && (u >> 1) < LOADS && more) issue_one(cur ^ 1, k0 + BKV, u >> 1);
        s[u & 1] = mfma32(kf[u], qf[u >> 1], s[u & 1]);
      }
      // s[kb][r] holds key k0 + 32kb + 16(r/8) + 8hi + r%8
      const bool interior = !has_mask && (k0 + BKV - 1 <= P + qw) && (k0 + BKV <= Tk);   // wave-uniform
      if (!interior) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t w = live_word(kb ? mw1 : mw0, k0 + 32 * kb);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((w >> (16 * (r >> 3) + (r & 7))) & 1u)) s[kb][r] = -INFINITY;
        }
      }
      if (mode == 1 || (mode == 0 && __any(m == -INFINITY))) {   // maxima wanted (uniform condition)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
        if (mode == 1) m = fmaxf(m, mx);
        else if (m == -INFINITY) m = mx;   // the query's first live keys: nothing accumulated yet
      }
      // (mode 1 still runs the value product below; its O is discarded)
      const float ms = m == -INFINITY ? 0.f : m;
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pf[kb * 2 + half][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][half * 8 + e], sl2, -ms));
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {pf[kb * 2 + half][e], pf[kb * 2 + half][e + 1]};
            if (kb) l1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l1, false);
            else l0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l0, false);
          }
        }
      // O^T += V^T . P^T; step ks covers keys 32(ks/2) + 16(ks%2) + 8hi + 0..7
      // step u = (ks, j) = (u / 4, u % 4); V^T fragments read two steps ahead
      auto vfrag = [&](int u) {
        const int ks = u >> 2, dv = (u & 3) * 32 + l32;
        const int c = (4 * (ks >> 1) + 2 * (ks & 1) + hi) ^ sw8(dv);
        return *(const bf16x8*)(sb + ST_VT + dv * 64 + (c << 3));
      };
      bf16x8 vf[16];
      vf[0] = vfrag(0);
      vf[1] = vfrag(1);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (u + 2 < 16) vf[u + 2] = vfrag(u + 2);
        o[u & 3] = mfma32(vf[u], pf[u >> 2], o[u & 3]);
      }
    };
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile(kt, std::integral_constant<int, 0>());
      if (kt + 1 < ntiles) tile(kt + 1, std::integral_constant<int, 1>());
    }
    l = l0 + l1;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // the stages are free for another pass
    if (mode == 0) {
      // a query whose sum left [0, 2^64) ran past its fixed max: exact two-pass
      // redo of the whole workgroup, decided through a flag in the (now idle) stage memory
      int* flag = (int*)smem;
      if (tid == 0) flag[0] = 0;
      __syncthreads();
      const float lsum = l + __shfl_xor(l, 32);
      if (__any(!(lsum < LSUM_MAX)) && lane == 0) flag[0] = 1;
      __syncthreads();
      const bool redo = flag[0] != 0;
      __syncthreads();   // every wave has read the flag before stage 0 is reloaded
      if (!redo) break;
      mode = 1;
      m = -INFINITY;
    } else if (mode == 1) {
      mode = 2;
    } else {
      break;
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (a.oq) {
    // e4m3 output for the next projection: the (query, head) row's 128 values
    // are this lane's 64 and those of lane ^ 32, one scale group
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[j][r] = __uint_as_float((uint32_t)f2bf(o[j][r] * inv) << 16);
        amax = fmaxf(amax, fabsf(o[j][r]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    e4m3_quotients(amax, true, [&](const float sc, auto quo) {
      if (q_ok) {
        const int64_t row = (int64_t)b * T + qi;
        uint8_t* op = a.oq + row * ((int64_t)H * 128) + h * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float v0 = o[j][r], v1 = o[j][r + 1], v2 = o[j][r + 2], v3 = o[j][r + 3];
            uint32_t code = 0u;
            if (sc != 0.f)
              code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                  quo(v2), quo(v3), __builtin_amdgcn_cvt_pk_fp8_f32(quo(v0), quo(v1), 0, false), true);
            *(uint32_t*)(op + j * 32 + row32(r, lane)) = code;
          }
        if (hi == 0) a.os[row * H + h] = sc;
      }
    });
    continue;
  }
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
  }   // zigzag tiles
}

// fp32 path: one wave per (query, head); lanes split the feature dims.
__global__ __launch_bounds__(64) void prefill_attn_f32_kernel(PrefillAttnArgs a) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int T = a.T, Tp = a.Tp, H = a.H, Tk = a.P + T;
  const int64_t bh = (int64_t)b * H + h;
  const float* Q = (const float*)a.q + ((int64_t)b * T + s) * H * 192 + h * 192;
  const float* KN = (const float*)a.kn + bh * Tp * 128;
  const float* VT = (const float*)a.vt + bh * 128 * Tp;
  const float* KP = (const float*)a.kpe + (int64_t)b * Tp * 64;
  const float q0 = Q[lane], q1 = Q[lane + 64], q2 = Q[lane + 128];
  const int W = (Tk + 31) >> 5;
  const uint32_t* mrow = a.mask ? a.mask + ((int64_t)b * T + s) * W : nullptr;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t = 0; t <= a.P + s; ++t) {
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
  const int nq = (a.T + BQ - 1) / BQ, pairs = a.B * a.H;
  const unsigned grid = 8u * (unsigned)((pairs + 7) / 8) * (unsigned)((nq + 1) / 2);
  prefill_attn_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn_f32(const PrefillAttnArgs& a, hipStream_t s) {
  dim3 grid(a.T, a.H, a.B);
  prefill_attn_f32_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
