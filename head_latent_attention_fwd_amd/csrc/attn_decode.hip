// Latent-absorbed single-token decode attention (DeepSeek-V3.2-Exp · Sparse
// attention, "Explanation": a single decoded token scores the cached latent
// directly; DeepSeek-V3.2-Exp · Output projection page at p = 1000).
//
// With kv_b's key half folded into the query, every head of sequence b scores
// the same cache rows C_t = [latent 512 | rope key 64]:
//   z[h, t] = scale * (q_lat[h] . C_t),  o_lat[h] = sum_t softmax_t(z[h]) C_t[:512]
// so one cache tile in LDS serves all heads of a workgroup.
//
// Workgroup = (sequence b, group of 64 heads); the head groups of one
// sequence are placed on the same XCD so the second read of the cache comes
// from that XCD's L2. Cache tiles of 32 keys move HBM -> LDS with 16-byte
// direct-to-LDS buffer loads through a 3-stage ring (two tiles in flight).
// Wave (hb, dh) = (wave & 1, wave >> 1) serves heads 32hb..32hb+31:
//   scores  S^T[t, h] = C[t, :] . Q^T[:, h]     each wave of a pair takes one half
//           of the 576 contracted dims (its half of Q stays in registers) and
//           the pair adds the two fp32 partials through LDS, in the same order;
//   values  O^T[d, h] += C^T[d, t] . P^T[t, h]  for the wave's 256 latent dims,
// both on v_mfma_f32_32x32x16_bf16 (C^T read with ds_read_b64_tr_b16). A lane's
// score results are 16 keys of one head, which are exactly the k slots the
// value product needs from P^T, so the probabilities stay in registers.
//
// Softmax: the running max of a head is fixed at its first live tile and
// later tiles add exp2(z - m) <= 2^LAZY, so the accumulators are never
// rescaled inside the loop. If a later score exceeds m + LAZY (a logit jump
// of ~44 nats) the workgroup recomputes its output in two passes: exact
// maxima first, then the accumulation with those maxima.
//
// Selected keys: with an index list the workgroup first compacts the row's
// live positions into LDS (ballot ranks, list order kept), padded with the
// last one, and tile row r then loads cache row keys[k0 + r] instead of k0 + r;
// everything after the loads is the dense path over nkeys = #live keys. The
// same kernel serves a prefill in the absorbed form, one query row per token.
//
// LDS stage: latent rows [32][1024 B] then rope rows [32][128 B]. The 16-byte
// chunks of latent row r are XOR-permuted within aligned groups of 16 by
// ((r & 3) << 2) | ((r >> 2) & 3) and those of rope row r by (r >> 1) & 7, so
// the row reads of the scores and the transposed reads of the values are free
// of bank conflicts. The stages are distinct LDS objects and every access
// names its stage statically, so the compiler can tell the reads of one stage
// from the loads in flight into the others.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int DKT = 32;                 // keys per tile
constexpr int DROW = 576;               // elements per cache row
constexpr int DLAT = DKT * 512;         // latent region of a stage (elements)
constexpr int DSTAGE = DKT * DROW;      // elements per stage
constexpr float LAZY = 64.f;            // log2-domain headroom over the fixed running max

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swl(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ v4s read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}

struct DecodeCtx {
  __amdgpu_buffer_rsrc_t rsrc;   // raw buffer over the cache rows of sequence b
  int nkeys, ntiles, wave, lane, hi, dh;
  float sl2;
  float* xs;                     // [2][4 waves][16][64] partial-score exchange
  bool sparse;                   // tile rows from `keys` (else keys 0..nkeys-1)
  const __attribute__((address_space(3))) int* keys;   // compacted selected positions
};

constexpr int KEYS_LDS = DECODE_TOPK_MAX + 4 * DKT;   // room for the tiles issued past the end

__device__ __forceinline__ void load_lds16(const DecodeCtx& c, uint16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0,
                                           0);
}

// Loads tile kt into stage st (9 loads per thread): latent instruction i of
// wave w fills row 8w + i (lane = physical chunk); the rope instruction of wave
// w fills rows 8w..8w+7 (8 chunks each). Rows past the last key repeat it
// (their scores are masked).
__device__ __forceinline__ void issue_tile(const DecodeCtx& c, uint16_t* st, int kt) {
  const int k0 = kt * DKT;
  if (c.sparse) {   // cache rows from the compacted list (entries past nkeys repeat the last key)
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
    const int t = min(k0 + r, c.nkeys - 1);
    load_lds16(c, st + r * 512, (c.lane ^ swl(r)) << 4, t * (DROW * 2));
  }
  const int r = 8 * c.wave + (c.lane >> 3);
  const int t = min(k0 + r, c.nkeys - 1);
  load_lds16(c, st + DLAT + c.wave * 512, t * (DROW * 2) + 1024 + (((c.lane & 7) ^ swr(r)) << 4), 0);
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
template <bool SCORES_ONLY>
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
  auto step = [&](int kt, const uint16_t* st, uint16_t* next) {
    __asm__ volatile("s_waitcnt vmcnt(9)" ::: "memory");   // tile kt landed, kt + 1 may be in flight
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    issue_tile(c, next, kt + 2);   // into the stage tile kt - 1 used

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

template <bool SPARSE>
__global__ __launch_bounds__(256, 1) void decode_attn_kernel(DecodeAttnArgs a, int n_hg) {
  __shared__ __attribute__((aligned(16))) uint16_t st0[DSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t st1[DSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t st2[DSTAGE];
  __shared__ __attribute__((aligned(16))) float xs[2 * 4 * 16 * 64];
  __shared__ __attribute__((aligned(16))) int keys[SPARSE ? KEYS_LDS : 4];
  __shared__ int wcount[4];
  __shared__ int s_over;

  const int tid = threadIdx.x;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  // query row q; its cache sequence b and last key P
  const int hg = loc % n_hg, q = (loc / n_hg) * 8 + xcd;
  if (q >= a.B) return;
  const int b = SPARSE && a.rows_per_seq > 0 ? q / a.rows_per_seq : q;
  const int P = SPARSE && a.rows_per_seq > 0 ? q - b * a.rows_per_seq : a.cache_len[b];
  DecodeCtx c;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.dh = c.wave >> 1;
  c.hi = c.lane >> 5;
  c.xs = xs;
  c.sl2 = a.scale * 1.4426950408889634f;
  c.sparse = SPARSE;
  c.keys = (const __attribute__((address_space(3))) int*)keys;
  c.nkeys = (P >= 0 && P < a.max_len) ? P + 1 : 0;
  if (SPARSE) {   // live listed positions t <= P, compacted in list order
    const int32_t* row = a.idx + (int64_t)q * a.topk;
    int base = 0;
    for (int j0 = 0; j0 < a.topk; j0 += 256) {
      const int j = j0 + tid;
      const int t = j < a.topk ? row[j] : -1;
      const bool ok = c.nkeys > 0 && t >= 0 && t <= P;
      const uint64_t bal = __ballot(ok);
      if (c.lane == 0) wcount[c.wave] = __popcll(bal);
      __syncthreads();
      int off = base;
      for (int w = 0; w < c.wave; ++w) off += wcount[w];
      if (ok) keys[off + __popcll(bal & ((1ull << c.lane) - 1))] = t;
      base += wcount[0] + wcount[1] + wcount[2] + wcount[3];
      __syncthreads();
    }
    c.nkeys = base;
    const int last = base > 0 ? keys[base - 1] : 0;
    for (int j = base + tid; j < KEYS_LDS; j += 256) keys[j] = last;
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
  if (c.ntiles > 0) over = attn_pass<false>(c, st0, st1, st2, qf, m, l, o);
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
    attn_pass<true>(c, st0, st1, st2, qf, m, l, o);
    attn_pass<false>(c, st0, st1, st2, qf, m, l, o);
  }
  // o_lat[b, head, 256 dh + 32 dt + 8 rg + 4 hi + 0..3]
  l += __shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.oq) {
    // e4m3 output: dims [256 dh + 128 g2, +128) are one group, held by this
    // lane (dt = 4 g2 .. 4 g2 + 3) and lane ^ 32
    const int64_t row = (int64_t)q * a.H + head;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      float amax = 0.f;
#pragma unroll
      for (int dt = 4 * g2; dt < 4 * g2 + 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o[dt][r] = __uint_as_float((uint32_t)f2bf(o[dt][r] * inv) << 16);
          amax = fmaxf(amax, fabsf(o[dt][r]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float sc = amax / 448.0f;
      uint8_t* oq = a.oq + row * 512 + 256 * c.dh + 4 * c.hi;
#pragma unroll
      for (int dt = 4 * g2; dt < 4 * g2 + 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const float v0 = o[dt][4 * rg], v1 = o[dt][4 * rg + 1], v2 = o[dt][4 * rg + 2], v3 = o[dt][4 * rg + 3];
          uint32_t code = 0u;
          if (sc != 0.f)
            code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                v2 / sc, v3 / sc, __builtin_amdgcn_cvt_pk_fp8_f32(v0 / sc, v1 / sc, 0, false), true);
          *(uint32_t*)(oq + 32 * dt + 8 * rg) = code;
        }
      if (c.hi == 0) a.os[row * 4 + 2 * c.dh + g2] = sc;
    }
    return;
  }
  uint16_t* out = (uint16_t*)a.olat + ((int64_t)q * a.H + head) * 512 + 256 * c.dh + 4 * c.hi;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      *(uint2*)(out + 32 * dt + 8 * rg) = make_uint2(pack_bf16x2(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv),
                                                     pack_bf16x2(o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv));
}

}  // namespace

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s) {
  const int n_hg = a.H / 64;
  const unsigned grid = 8u * (unsigned)((a.B + 7) / 8) * (unsigned)n_hg;
  if (a.idx) {
    if (a.topk <= 0 || a.topk > DECODE_TOPK_MAX || a.rows_per_seq < 0) return hipErrorInvalidValue;
    decode_attn_kernel<true><<<grid, 256, 0, s>>>(a, n_hg);
  } else {
    if (a.rows_per_seq != 0) return hipErrorInvalidValue;
    decode_attn_kernel<false><<<grid, 256, 0, s>>>(a, n_hg);
  }
  return hipGetLastError();
}

}  // namespace mla
