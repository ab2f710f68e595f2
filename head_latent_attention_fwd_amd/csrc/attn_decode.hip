// Latent-absorbed single-token decode attention (DeepSeek-V3.2-Exp · Sparse
// attention, "Explanation": a single decoded token scores the cached latent
// directly; DeepSeek-V3.2-Exp · Output projection page at p = 1000).
//
// With kv_b's key half folded into the query, every head of row q scores the
// same cache rows C_t = [latent 512 | rope key 64]:
//   z[h, t] = scale * (q_lat[h] . C_t),  o_lat[h] = sum_t softmax_t(z[h]) C_t[:512]
// so one cache tile in LDS serves every head of the row.
//
// Workgroup = (row q, group of 64 heads, key run j), four waves. The key
// range of a row is cut into `splits` runs of whole 32-key tiles (as many as
// it takes for rows x head groups x runs to fill the chip); with one run the
// workgroup writes the normalised o_lat, otherwise its normalised partial and
// its log2-sum-exp, which the consumer merges in run order
// (launch_decode_combine or the un-absorb kernel). All workgroups of a row are
// placed on one XCD, so the second head group's read of a cache tile comes
// from that XCD's L2.
//
// Wave (hb, dh) = (wave & 1, wave >> 1) serves heads 32hb..32hb+31 of the group:
//   scores  S^T[t, h] = C[t, :] . Q^T[:, h]   each wave of the pair (hb, 0) /
//           (hb, 1) takes one half of the 576 contracted dims (its half of Q
//           stays in registers) and the pair adds the two fp32 partials
//           through LDS, in the same order;
//   values  O^T[d, h] += C^T[d, t] . P^T[t, h] for the wave's 256 latent dims,
// both on v_mfma_f32_32x32x16_bf16 (C^T read with ds_read_b64_tr_b16). A
// lane's score results are 16 keys of one head, exactly the k slots the value
// product needs from P^T, so the probabilities stay in registers. Cache tiles
// move HBM -> LDS with 16-byte direct-to-LDS buffer loads through a 3-stage
// ring (two tiles in flight).
//
// Softmax: the running max of a head is fixed at its first live tile and
// later tiles add exp2(z - m) <= 2^LAZY, so the accumulators are never
// rescaled inside the loop. If a later score exceeds m + LAZY (a logit jump
// of ~44 nats) the workgroup recomputes its output in two passes: exact
// maxima first, then the accumulation with those maxima.
//
// Selected keys: launch_decode_compact first turns each row's index list into
// its ascending, duplicate-free list of live positions; the workgroup copies
// its split's part of that list to LDS (padded with its last key) and tile row
// r loads cache row keys[k0 + r]. The same kernel serves a prefill in the
// absorbed form, one query row per token.
//
// e4m3 weights (QLAT): kv_b is an e4m3 Linear whose input, the latent, is
// quantised in dynamic 1x128 groups (Kimi K2 · Down projection,
// quantization_config). The absorbed product therefore sees each latent as
// its dequantised value: once a tile has landed, the workgroup replaces every
// latent 128-group of the tile in LDS by scale * e4m3(x / scale) (scale =
// amax / 448 in fp32, quotient from the correctly rounded reciprocal plus one
// residual correction), rounded to bf16. The rope key is not an input of kv_b
// and is used as cached.
//
// LDS stage: latent rows [32][1024 B] then rope rows [32][128 B]. The 16-byte
// chunks of latent row r are XOR-permuted within aligned groups of 16 by
// ((r & 3) << 2) | ((r >> 2) & 3) and those of rope row r by (r >> 1) & 7, so
// the row reads of the scores and the transposed reads of the values are free
// of bank conflicts. The stages are distinct LDS objects and every access
// names its stage statically, so the compiler can tell the reads of one stage
// from the loads in flight into the others.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int DKT = 32;                 // keys per tile
constexpr int DROW = 576;               // elements per cache row
constexpr int DLAT = DKT * 512;         // latent region of a stage (elements)
constexpr int DSTAGE = DKT * DROW;      // elements per stage
constexpr float LAZY = 64.f;            // log2-domain headroom over the fixed running max
constexpr int KEYS_LDS = DECODE_TOPK_MAX + 4 * DKT;   // a split's keys plus the tiles issued past its end

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swl(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ v4s read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}

struct DecodeCtx {
  __amdgpu_buffer_rsrc_t rsrc;   // raw buffer over the cache rows of the row's sequence
  int k0, nkeys, ntiles, wave, lane, hi, dh;   // keys k0 .. k0 + nkeys - 1 (dense) or list slots (sparse)
  float sl2;
  float* xs;                     // [2][4 waves][16][64] partial-score exchange
  bool sparse;                   // tile rows from `keys` (else keys k0..k0+nkeys-1)
  const __attribute__((address_space(3))) int* keys;   // the run's selected positions
};

__device__ __forceinline__ void load_lds16(const DecodeCtx& c, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0,
                                           0);
}

// Loads tile kt of the run into stage st (9 loads per thread): latent
// instruction i of wave w fills row 8w + i (lane = physical chunk); the rope
// instruction of wave w fills rows 8w..8w+7 (8 chunks each). Rows past the
// run's last key repeat it (their scores are masked).
__device__ __forceinline__ void issue_tile(const DecodeCtx& c, uint16_t* st, int kt) {
  const int k0 = kt * DKT;
  if (c.sparse) {   // cache rows from the run's list (slots past its end repeat the last key)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * c.wave + i;
      load_lds16(c, st + r * 512, (c.lane ^ swl(r)) << 4, __builtin_amdgcn_readfirstlane(c.keys[k0 + r]) * (DROW * 2));
    }
    const int r = 8 * c.wave + (c.lane >> 3);
    const int t = c.keys[k0 + r];
    load_lds16(c, st + DLAT + c.wave * 512, t * (DROW * 2) + 1024 + (((c.lane & 7) ^ swr(r)) << 4), 0);
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * c.wave + i;
    const int t = c.k0 + min(k0 + r, c.nkeys - 1);
    load_lds16(c, st + r * 512, (c.lane ^ swl(r)) << 4, t * (DROW * 2));
  }
  const int r = 8 * c.wave + (c.lane >> 3);
  const int t = c.k0 + min(k0 + r, c.nkeys - 1);
  load_lds16(c, st + DLAT + c.wave * 512, t * (DROW * 2) + 1024 + (((c.lane & 7) ^ swr(r)) << 4), 0);
}

// e4m3 view of a tile's latent: thread (row r = tid / 8, group g = (tid / 2) % 4,
// half hf = tid % 2) takes the 8 chunks 16 g + 8 hf .. + 7 of row r; the two
// halves of a group are neighbouring lanes.
__device__ __forceinline__ void quant_dequant_tile(uint16_t* st, int tid) {
  const int r = tid >> 3, g = (tid >> 1) & 3, hf = tid & 1;
  uint4 v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = 8 * hf + i;   // chunk within the group's aligned 16
    v[i] = *(const uint4*)(st + r * 512 + ((16 * g + (ch ^ swl(r))) << 3));
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xffff0000u))));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  e4m3_quotients(amax, true, [&](const float s, auto quo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xffff0000u);
        const int code = __builtin_amdgcn_cvt_pk_fp8_f32(quo(x0), quo(x1), 0, false);
        const float2v d = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
        o[e] = pack_bf16x2(d[0] * s, d[1] * s);
      }
      const int ch = 8 * hf + i;
      *(uint4*)(st + r * 512 + ((16 * g + (ch ^ swl(r))) << 3)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  });
}

// Partial scores of one tile over the wave's half of the contracted dims:
// dh = 0 takes latent chunks 0..35, dh = 1 latent chunks 36..63 and the rope
// chunks; chunk 2kk + hi meets query fragment kk.
template <int DH>
__device__ __forceinline__ floatx16 partial_scores(const uint16_t* st, int srow, int hi, const bf16x8 (&qf)[18]) {
  auto frag = [&](int kk) {
    const int c = 36 * DH + 2 * kk;   // + hi
    if (c < 64) {
      const int f = swl(srow) ^ hi;
      return *(const bf16x8*)(st + srow * 512 + ((c & ~15) << 3) + (((c & 15) ^ f) << 3));
    }
    return *(const bf16x8*)(st + DLAT + srow * 64 + (((c - 64) ^ (swr(srow) ^ hi)) << 3));
  };
  // two accumulators (even / odd k steps) so consecutive MFMAs are independent;
  // fragments are read two steps ahead
  floatx16 sa, sb;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sa[r] = 0.f;
    sb[r] = 0.f;
  }
  bf16x8 f0 = frag(0), f1 = frag(1), f2;
#pragma unroll
  for (int kk = 0; kk < 18; ++kk) {
    if (kk + 2 < 18) f2 = frag(kk + 2);
    if (kk & 1) sb = mfma32(f0, qf[kk], sb);
    else sa = mfma32(f0, qf[kk], sa);
    f0 = f1;
    f1 = f2;
  }
  return sa + sb;
}

// One pass over the sequence. SCORES_ONLY: m becomes the exact per-head max.
// Otherwise accumulates o and l against m (set at the first live tile when it
// is -inf); returns true when a score exceeded m + LAZY (results invalid).
template <bool SCORES_ONLY, bool QLAT>
__device__ __forceinline__ bool attn_pass(const DecodeCtx& c, uint16_t* st0, uint16_t* st1, uint16_t* st2,
                                          const bf16x8 (&qf)[18], float& m, float& l, floatx16 (&o)[8]) {
  const int lane = c.lane, l32 = lane & 31, hi = c.hi;
  // transposed reads: 16-lane group q reads rows 16 s + 4 (q >> 1) + 8 e + (lane % 16) / 4,
  // columns 256 dh + 32 dt + 16 (q & 1) + 4 (lane % 4)
  const int q4 = lane >> 4, L = lane & 15;
  const int trow = 4 * (q4 >> 1) + (L >> 2);
  const int tx = 2 * (q4 & 1) + ((L >> 1) & 1);
  int toff[2][4];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      const int r = trow + 8 * e;
      toff[e][d4] = r * 512 + 256 * c.dh + (((4 * d4 + tx) ^ swl(r)) << 3) + 4 * (L & 1);
    }
  bool over = false;
  if (!SCORES_ONLY) {
    l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  }
  auto step = [&](int kt, uint16_t* st, uint16_t* next) {
    __asm__ volatile("s_waitcnt vmcnt(9)" ::: "memory");   // tile kt landed, kt + 1 may be in flight
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    issue_tile(c, next, kt + 2);   // into the stage tile kt - 1 used
    if (QLAT) {   // replace the landed tile's latent by its dequantised e4m3 value
      quant_dequant_tile(st, 64 * c.wave + lane);
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS writes only: the loads stay in flight
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    }

    floatx16 sa = c.dh ? partial_scores<1>(st, l32, hi, qf) : partial_scores<0>(st, l32, hi, qf);
    float* xw = c.xs + (kt & 1) * (4 * 16 * 64);
#pragma unroll
    for (int r = 0; r < 16; ++r) xw[(c.wave * 16 + r) * 64 + lane] = sa[r];
    // exchange barrier: LDS writes only (a __syncthreads here would also drain the tile loads)
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    const int k0 = kt * DKT;
    float part[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = xw[((c.wave ^ 2) * 16 + r) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = (c.dh ? part[r] + sa[r] : sa[r] + part[r]) * c.sl2;   // first + second half
    if (k0 + DKT > c.nkeys) {   // wave-uniform: the tile runs past the last key
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k0 + row32(r, lane) >= c.nkeys) sa[r] = -INFINITY;
    }
    float mx = sa[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sa[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (SCORES_ONLY) {
      m = fmaxf(m, mx);
      return;
    }
    if (m == -INFINITY) m = mx;   // first live keys of this head: nothing accumulated yet
    over |= mx > m + LAZY;
    bf16x8 pf[2];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(sa[r] - m);   // masked keys: exp2(-inf) = 0
      rs += p;
      pf[r >> 3][r & 7] = (__bf16)p;
    }
    l += rs;
    // value product, step j = (key half j / 8, d tile j % 8): consecutive MFMAs
    // update different accumulators; C^T fragments read two steps ahead
    auto vfrag = [&](int j) {
      const int dt = j & 7, imm = 16 * (j >> 3) * 512 + 128 * (dt >> 2);
      const v4s lo = read_tr(st + toff[0][dt & 3] + imm), up = read_tr(st + toff[1][dt & 3] + imm);
      return __builtin_bit_cast(bf16x8, (v8s){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    bf16x8 vb0 = vfrag(0), vb1 = vfrag(1), vb2;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j + 2 < 16) vb2 = vfrag(j + 2);
      o[j & 7] = mfma32(vb0, pf[j >> 3], o[j & 7]);
      vb0 = vb1;
      vb1 = vb2;
    }
  };
  // The loop runs whole rounds of three tiles and always keeps two tiles in
  // flight; tiles past the end hold copies of the last key (all masked, p = 0)
  // and cost a little math. Straight-line rounds let the compiler's own LDS
  // waits see which stage each load targets.
  issue_tile(c, st0, 0);
  issue_tile(c, st1, 1);
  for (int kt = 0; kt < c.ntiles; kt += 3) {
    step(kt, st0, st2);
    step(kt + 1, st1, st0);
    step(kt + 2, st2, st1);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // every wave is done with the stages and the exchange buffer
  return over;
}

template <bool SPARSE, bool QLAT>
__global__ __launch_bounds__(256, 1) void decode_attn_kernel(DecodeAttnArgs a, int n_hg) {
  __shared__ __attribute__((aligned(16))) uint16_t st0[DSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t st1[DSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t st2[DSTAGE];
  __shared__ __attribute__((aligned(16))) float xs[2 * 4 * 16 * 64];
  __shared__ __attribute__((aligned(16))) int keys[SPARSE ? KEYS_LDS : 4];
  __shared__ int s_over;

  const int tid = threadIdx.x;
  const int NS = a.splits;
  // workgroup -> (row q, head group hg, run j); all of a row's workgroups on one XCD
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int j = loc % NS, hg = (loc / NS) % n_hg, q = (loc / (NS * n_hg)) * 8 + xcd;
  if (q >= a.R) return;
  const int b = a.rows_per_seq > 0 ? q / a.rows_per_seq : q;
  const int P = a.rows_per_seq > 0 ? q - b * a.rows_per_seq : a.cache_len[b];
  const bool valid = P >= 0 && P < a.max_len;
  DecodeCtx c;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.dh = c.wave >> 1;
  c.hi = c.lane >> 5;
  c.xs = xs;
  c.sl2 = a.scale * 1.4426950408889634f;
  c.sparse = SPARSE;
  c.keys = (const __attribute__((address_space(3))) int*)keys;
  // the row's keys (positions 0..P, or its compacted list) cut into NS runs of whole tiles
  const int n_all = !valid ? 0 : SPARSE ? a.nkeys[q] : P + 1;
  const int tiles_all = (n_all + DKT - 1) / DKT, tps = (tiles_all + NS - 1) / NS;
  const int kb = min(n_all, j * tps * DKT), ke = min(n_all, (j + 1) * tps * DKT);
  c.k0 = SPARSE ? 0 : kb;
  c.nkeys = ke - kb;
  if (SPARSE) {   // this run's slots of the compacted list, padded with its last key
    const int32_t* row = a.keys + (int64_t)q * a.kstride;
    const int last = c.nkeys > 0 ? row[ke - 1] : 0;
    for (int i = tid; i < KEYS_LDS; i += 256) keys[i] = i < c.nkeys ? row[kb + i] : last;
    __syncthreads();
  }
  c.ntiles = (c.nkeys + DKT - 1) / DKT;
  c.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)a.cache + (int64_t)b * a.max_len * DROW),
                                             (short)0, a.max_len * DROW * 2, BUF_DW3);
  const int head = hg * 64 + (c.wave & 1) * 32 + (c.lane & 31);

  // this wave's half of the query: B operand of the score product, dims 288 dh + 16 kk + 8 hi + 0..7
  bf16x8 qf[18];
  {
    const uint16_t* qp = (const uint16_t*)a.qlat + ((int64_t)q * a.H + head) * DROW + 288 * c.dh + 8 * c.hi;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 16 * kk));
  }
  if (tid == 0) s_over = 0;
  floatx16 o[8];
  float m = -INFINITY, l = 0.f;
  bool over = false;
  if (c.ntiles > 0) over = attn_pass<false, QLAT>(c, st0, st1, st2, qf, m, l, o);
  else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    __syncthreads();
  }
  if (over) s_over = 1;
  __syncthreads();
  if (s_over) {   // rare: exact maxima, then accumulate against them (no score can exceed them)
    m = -INFINITY;
    attn_pass<true, QLAT>(c, st0, st1, st2, qf, m, l, o);
    attn_pass<false, QLAT>(c, st0, st1, st2, qf, m, l, o);
  }
  // lane: head `head`, dims 256 dh + 32 dt + 8 rg + 4 hi + 0..3
  l += __shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t row = (int64_t)q * a.H + head;
  uint16_t* out = NS == 1 ? (uint16_t*)a.olat + row * 512 : (uint16_t*)a.part + ((int64_t)j * a.R * a.H + row) * 512;
  out += 256 * c.dh + 4 * c.hi;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      *(uint2*)(out + 32 * dt + 8 * rg) = make_uint2(pack_bf16x2(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv),
                                                     pack_bf16x2(o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv));
  if (NS > 1 && c.dh == 0 && c.hi == 0) a.lse[(int64_t)j * a.R * a.H + row] = l > 0.f ? m + __log2f(l) : -INFINITY;
}

// One workgroup per row: the listed positions t with 0 <= t <= last key of the
// row, ascending and without repeats. A list that is already ascending (after
// invalid entries are dropped) skips the bitonic sort.
__global__ __launch_bounds__(256) void decode_compact_kernel(const int32_t* __restrict__ idx, int topk,
                                                             const int32_t* __restrict__ cache_len, int rows_per_seq,
                                                             int max_len, int32_t* __restrict__ keys, int kstride,
                                                             int32_t* __restrict__ nkeys) {
  __shared__ int v[DECODE_TOPK_MAX];
  __shared__ int wcount[4];
  __shared__ int s_unsorted;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = rows_per_seq > 0 ? q / rows_per_seq : q;
  const int P = rows_per_seq > 0 ? q - b * rows_per_seq : cache_len[b];
  const bool valid = P >= 0 && P < max_len;
  int n2 = 1;
  while (n2 < topk) n2 <<= 1;
  const int32_t* src = idx + (int64_t)q * topk;
  if (tid == 0) s_unsorted = 0;
  for (int i = tid; i < n2; i += 256) {
    const int t = i < topk ? src[i] : -1;
    v[i] = valid && t >= 0 && t <= P ? t : INT_MAX;
  }
  __syncthreads();
  bool uns = false;
  for (int i = tid; i + 1 < n2; i += 256) uns |= v[i] > v[i + 1];
  if (uns) s_unsorted = 1;
  __syncthreads();
  if (s_unsorted) {
    for (int k = 2; k <= n2; k <<= 1)
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < n2; i += 256) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const int x = v[i], y = v[ixj];
            if ((x > y) == ((i & k) == 0)) {
              v[i] = y;
              v[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
  }
  // keep the first of each run of equal live positions, in order
  int32_t* dst = keys + (int64_t)q * kstride;
  int base = 0;
  for (int i0 = 0; i0 < n2; i0 += 256) {
    const int i = i0 + tid;
    const int x = i < n2 ? v[i] : INT_MAX;
    const bool keep = x != INT_MAX && (i == 0 || v[i - 1] != x);
    const uint64_t bal = __ballot(keep);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wcount[w];
    if (keep) dst[off + __popcll(bal & ((1ull << lane) - 1))] = x;
    base += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    __syncthreads();
  }
  if (tid == 0) nkeys[q] = base;
}

// o_lat[r] = sum_j w_j part[j][r] / sum_j w_j with w_j = exp2(lse[j][r] - max_j lse), in split order
// (rows with every lse = -inf get 0). One thread per 8 dims of a row.
__global__ __launch_bounds__(256) void decode_combine_kernel(const uint16_t* __restrict__ part,
                                                             const float* __restrict__ lse, int splits, int64_t rows,
                                                             uint16_t* __restrict__ olat) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = i >> 6;
  if (r >= rows) return;
  const int c8 = (int)(i & 63) * 8;
  float mx = -INFINITY;
  for (int j = 0; j < splits; ++j) mx = fmaxf(mx, lse[j * rows + r]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, den = 0.f;
  if (mx != -INFINITY) {
    for (int j = 0; j < splits; ++j) {
      const float w = __builtin_amdgcn_exp2f(lse[j * rows + r] - mx);
      den += w;
      const uint4 u = *(const uint4*)(part + ((int64_t)j * rows + r) * 512 + c8);
      const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * __uint_as_float(p[e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(p[e] & 0xffff0000u);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *(uint4*)(olat + r * 512 + c8) = make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                              pack_bf16x2(acc[2] * inv, acc[3] * inv),
                                              pack_bf16x2(acc[4] * inv, acc[5] * inv),
                                              pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

}  // namespace

int decode_splits(int rows, int H, int max_keys) {
  const int n_hg = (H + 63) / 64;
  const int wgs = rows * n_hg;
  int ns = wgs >= 256 ? 1 : (256 + wgs - 1) / wgs;
  const int tiles = (max_keys + DKT - 1) / DKT;
  const int cap = tiles / 4 > 1 ? tiles / 4 : 1;   // at least ~4 tiles per split
  if (ns > cap) ns = cap;
  if (ns > DECODE_MAX_SPLITS) ns = DECODE_MAX_SPLITS;
  return ns;
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.H % 64) return hipErrorInvalidValue;
  const int n_hg = a.H / 64;
  if (a.splits < 1 || a.splits > DECODE_MAX_SPLITS || (a.splits > 1 && (!a.part || !a.lse)) ||
      (a.splits == 1 && !a.olat))
    return hipErrorInvalidValue;
  const unsigned grid = 8u * (unsigned)((a.R + 7) / 8) * (unsigned)n_hg * (unsigned)a.splits;
  if (a.keys) {
    if (!a.nkeys || a.kstride < 0 || a.kstride > DECODE_TOPK_MAX) return hipErrorInvalidValue;
    if (a.quant_latent) decode_attn_kernel<true, true><<<grid, 256, 0, s>>>(a, n_hg);
    else decode_attn_kernel<true, false><<<grid, 256, 0, s>>>(a, n_hg);
  } else {
    if (a.rows_per_seq != 0) return hipErrorInvalidValue;
    if (a.quant_latent) decode_attn_kernel<false, true><<<grid, 256, 0, s>>>(a, n_hg);
    else decode_attn_kernel<false, false><<<grid, 256, 0, s>>>(a, n_hg);
  }
  return hipGetLastError();
}

hipError_t launch_decode_compact(const int32_t* idx, int topk, const int32_t* cache_len, int rows_per_seq, int rows,
                                 int max_len, int32_t* keys, int kstride, int32_t* nkeys, hipStream_t s) {
  if (topk <= 0 || topk > DECODE_TOPK_MAX || kstride < topk) return hipErrorInvalidValue;
  decode_compact_kernel<<<rows, 256, 0, s>>>(idx, topk, cache_len, rows_per_seq, max_len, keys, kstride, nkeys);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const void* part, const float* lse, int splits, int64_t rows, void* olat,
                                 hipStream_t s) {
  const int64_t threads = rows * 64;
  decode_combine_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>((const uint16_t*)part, lse, splits, rows,
                                                                         (uint16_t*)olat);
  return hipGetLastError();
}

}  // namespace mla

// ---------------------------------------------------------------------------
// Library-held scratch for the allocation-free variant of the decode attention
// (callers that cannot allocate: code under graph capture, tight serving
// loops). Each GPU the library runs on holds its own copy of this array until
// the process ends; host code never passes the array's name to a kernel (on
// the host it is only a stand-in), only the device address that
// hipGetSymbolAddress returns for the current device.
namespace {
static __device__ __align__(256) uint8_t scratch[mla::DECODE_SCRATCH_BYTES];
}  // namespace

namespace mla {

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {   // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace mla
