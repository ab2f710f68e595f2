// Latent-absorbed single-token decode attention (DeepSeek-V3.2-Exp · Sparse
// attention, "Explanation": a single decoded token scores the cached latent
// directly; DeepSeek-V3.2-Exp · Output projection page at p = 1000).
//
// With kv_b's key half folded into the query, every head of row q scores the
// same cache rows C_t = [latent 512 | rope key 64]:
//   z[h, t] = scale * (q_lat[h] . C_t),  o_lat[h] = sum_t softmax_t(z[h]) C_t[:512]
// so one cache tile in LDS serves every head of the row.
//
// Workgroup = (row q, group of 64 heads, key run j), eight waves in two roles
// (two waves per SIMD, one of each). The key range of a row is cut into
// `splits` runs of whole 32-key tiles (as many as it takes for rows x head
// groups x runs to fill the chip); with one run the workgroup writes the
// normalised o_lat, otherwise its normalised partial and its log2-sum-exp,
// which the consumer merges in run order (launch_decode_combine or the
// un-absorb kernel). All workgroups of a row are placed on one XCD, so the
// second head group's read of a cache tile comes from that XCD's L2.
//
//   score wave s (waves 0..3), heads 16 s .. 16 s + 15 of the group: the
//     whole 576-dim product S^T[t, h] = C[t, :] . Q^T[:, h] on
//     v_mfma_f32_16x16x32_bf16 (its query stays in registers), the softmax,
//     and the tile's probabilities P[h, t] (bf16) into an LDS buffer;
//   value wave v (waves 4..7), latent dims 128 v .. 128 v + 127 of every head
//     of the group: O^T[d, h] += C^T[d, t] . P^T[t, h] on
//     v_mfma_f32_32x32x16_bf16, one tile behind the score waves (C^T read with
//     ds_read_b64_tr_b16, P^T as 16-byte rows of the buffer).
// Cache tiles move HBM -> LDS by 16-byte direct-to-LDS loads through a
// 3-stage ring with two tiles in flight. A value wave reloads the 8 KB of the
// stage that only it reads (its 128 dims of the 32 rows) as soon as its own
// fragments of the tile are in registers; the score waves reload the rope
// rows right after the next barrier, once every score wave has read them. One
// barrier per tile orders it all.
//
// Softmax: the running max of a head stays at its first live tile's value
// while later tiles add exp2(z - m) <= 2^LAZY. A tile whose max exceeds
// m + LAZY (a logit jump of ~44 nats) moves m to that max; the score wave
// scales its row sum by exp2(m_old - m_new) and hands the same factor to the
// value waves with the tile's probabilities, which scale their accumulators
// before adding the tile (a wave-uniform branch taken only then).
//
// Selected keys: launch_decode_compact first turns each row's index list into
// its ascending, duplicate-free list of live positions; the workgroup copies
// its split's part of that list to LDS (padded with its last key) and tile row
// r loads cache row keys[k0 + r]. The same kernel serves a prefill in the
// absorbed form, one query row per token.
//
// e4m3 weights: kv_b is an e4m3 Linear whose input, the latent, is quantised
// in dynamic 1x128 groups (Kimi K2 · Down projection, quantization_config);
// with e4m3 weights the cache holds each latent in that quantised form (the
// norm pass writes it so, and it is a fixed point of the quantiser), so the
// same kernel serves both weight types. The rope key is not an input of kv_b.
//
// LDS stage: the latent as four 128-dim groups, each [32 rows][256 B], then
// the rope rows [32][128 B]. The 16-byte chunks of a latent group's row r are
// XOR-permuted by swl(r) and those of rope row r by (r >> 1) & 7 to keep the
// score waves' row reads and the value waves' transposed reads off shared
// banks.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int DKT = 32;                 // keys per tile
constexpr int DROW = 576;               // elements per cache row
constexpr int DGRP = DKT * 128;         // elements of one 128-dim latent group of a stage
constexpr int DLAT = 4 * DGRP;          // latent region of a stage (elements)
constexpr int DSTAGE = DKT * DROW;      // elements per stage
constexpr float LAZY = 64.f;            // log2-domain headroom over the running max
constexpr int KEYS_LDS = DECODE_TOPK_MAX + DKT;   // a split's keys plus the rest of its last tile

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

// 16-byte chunk permutation of latent row r (XOR of per-bit images 12, 1, 4, 2 of
// r's low four bits), chosen by timing candidates on gfx950 for both read
// patterns below: with it the 16x16x32 operand reads run at ~199 B/clk per CU,
// against ~126 for ((r & 3) << 2) | ((r >> 2) & 3), and the transposed reads
// are no slower.
__device__ __forceinline__ int swl(int r) {
  return ((r & 1) ? 12 : 0) ^ ((r & 2) ? 1 : 0) ^ ((r & 4) ? 4 : 0) ^ ((r & 8) ? 2 : 0);
}
__device__ __forceinline__ int swr(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ v4s read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
}

// x[l] combined with x[l ^ 16] and with x[l ^ 32] (VALU lane swaps, no LDS round trip)
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p);
}

// 16-byte direct-to-LDS load: lane l's bytes land at LDS byte address base + 16 l.
// Written as asm so that the compiler does not order later LDS reads behind
// it; the ring's explicit vmcnt waits do.
__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t base) {
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(base)
                   : "memory", "m0");
}

// LDS waits before a barrier: the wave's own LDS writes done and at most
// `ahead` of its direct loads still in flight (their counts are wave-uniform).
template <int N>
__device__ __forceinline__ void wait_tile(bool more) {
  if (more) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  else __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <bool SPARSE>
__global__ __launch_bounds__(512, 1) void decode_attn_kernel(DecodeAttnArgs a, int n_hg) {
  __shared__ __attribute__((aligned(16))) uint16_t stages[3 * DSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][64 * DKT];   // P[h][t] bf16, per tile parity
  __shared__ float fbuf[2][64];                                          // rescale factor per head
  __shared__ float s_l[64];
  __shared__ __attribute__((aligned(16))) int keys[SPARSE ? KEYS_LDS : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score = wave < 4;
  const int NS = a.splits;
  // workgroup -> (row q, head group hg, run j); all of a row's workgroups on one XCD
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int j = loc % NS, hg = (loc / NS) % n_hg, q = (loc / (NS * n_hg)) * 8 + xcd;
  if (q >= a.R) return;
  const int b = a.rows_per_seq > 0 ? q / a.rows_per_seq : q;
  const int P = a.rows_per_seq > 0 ? q - b * a.rows_per_seq : a.cache_len[b];
  const bool valid = P >= 0 && P < a.max_len;
  // the row's keys (positions 0..P, or its compacted list) cut into NS runs of whole tiles
  const int n_all = !valid ? 0 : SPARSE ? a.nkeys[q] : P + 1;
  const int tiles_all = (n_all + DKT - 1) / DKT, tps = (tiles_all + NS - 1) / NS;
  const int kb = min(n_all, j * tps * DKT), ke = min(n_all, (j + 1) * tps * DKT);
  const int nkeys = ke - kb, nt = (nkeys + DKT - 1) / DKT;
  if (SPARSE) {   // this run's slots of the compacted list, padded with its last key
    const int32_t* row = a.keys + (int64_t)q * a.kstride;
    const int last = nkeys > 0 ? row[ke - 1] : 0;
    for (int i = tid; i < KEYS_LDS; i += 512) keys[i] = i < nkeys ? row[kb + i] : last;
    __syncthreads();
  }
  const uint16_t* cache = (const uint16_t*)a.cache + (int64_t)b * a.max_len * DROW;
  // cache row of tile slot x of the run (slots past its end repeat its last key)
  auto key_row = [&](int x) { return SPARSE ? keys[x] : kb + min(x, nkeys - 1); };
  const float sl2 = a.scale * 1.4426950408889634f;
  const int64_t hrow0 = (int64_t)q * a.H + hg * 64;   // first (row, head) of the group

  if (score) {
    // ---------------- score wave s: heads 16 s + (lane % 16) ----------------
    const int s = wave, hl = 16 * s + (lane & 15), kq = lane >> 4;
    // query: B operand of the 16x16x32 product, dims 32 ks + 8 kq + 0..7
    bf16x8 qf[18];
    {
      const uint16_t* qp = (const uint16_t*)a.qlat + (hrow0 + hl) * DROW + 8 * kq;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = *(const bf16x8*)(qp + 32 * ks);
      // from here on the query registers count as written (one wait here, none per tile
      // behind the ring's loads)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) __asm__ volatile("" : "+v"(qf[ks]));
    }
    // rope rows of tile kt: rows 8 s + lane / 8, physical chunk lane % 8
    auto issue_rope = [&](int kt, uint16_t* st) {
      const int r = 8 * s + (lane >> 3);
      dma16(cache + (int64_t)key_row(kt * DKT + r) * DROW + 512 + (((lane & 7) ^ swr(r)) << 3),
            lds_addr(st + DLAT + s * 512));
    };
    float m = -INFINITY, l = 0.f;
    if (nt > 0) issue_rope(0, stages);
    if (nt > 1) issue_rope(1, stages + DSTAGE);
    int cur = 0;   // stage of tile i
    for (int i = 0; i <= nt; ++i) {
      wait_tile<1>(i + 1 < nt);
      barrier();
      // rope rows of tile i + 2 into the stage tile i - 1 used: every score wave read
      // them before this barrier, so they go out now, a whole tile ahead of their use
      const int nx = cur == 0 ? 2 : cur - 1;
      if (i + 2 < nt) issue_rope(i + 2, stages + nx * DSTAGE);
      uint16_t* st = stages + cur * DSTAGE;
      if (i < nt) {
        // A operand rows t = 16 tb + lane % 16, chunk 4 ks + kq of the 72 in a row
        auto afrag = [&](int tb, int ks) {
          const int t = 16 * tb + (lane & 15), c = 4 * ks + kq;
          if (ks < 16) return *(const bf16x8*)(st + (c >> 4) * DGRP + t * 128 + (((c & 15) ^ swl(t)) << 3));
          return *(const bf16x8*)(st + DLAT + t * 64 + (((c - 64) ^ swr(t)) << 3));
        };
        floatx4 acc[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[u][0][r] = acc[u][1][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) acc[tb][ks & 1] = mfma16(afrag(tb, ks), qf[ks], acc[tb][ks & 1]);
        // lane: head hl, keys 16 tb + 4 kq + r of the tile
        const int k0 = i * DKT;
        float z[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) z[4 * tb + r] = (acc[tb][0][r] + acc[tb][1][r]) * sl2;
        if (k0 + DKT > nkeys) {   // wave-uniform: the tile runs past the last key
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + 16 * (e >> 2) + 4 * kq + (e & 3) >= nkeys) z[e] = -INFINITY;
        }
        float mx = z[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
        mx = max_xor32(max_xor16(mx));
        float f = 1.f;
        if (m == -INFINITY) m = mx;   // first live keys of this head: nothing accumulated yet
        else if (mx > m + LAZY) {     // rare: move the max, rescale what is accumulated
          f = __builtin_amdgcn_exp2f(m - mx);
          l *= f;
          m = mx;
        }
        const float mref = m == -INFINITY ? 0.f : m;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(z[e] - mref);   // masked keys: exp2(-inf) = 0
          l += p[e];
        }
        uint16_t* pb = pbuf[i & 1] + hl * DKT;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {   // keys 16 tb + 4 kq .. +3: chunk 2 tb + kq / 2, half kq % 2
          const int ch = (2 * tb + (kq >> 1)) ^ ((hl >> 2) & 3);
          *(uint2*)(pb + (ch << 3) + 4 * (kq & 1)) =
              make_uint2(pack_bf16x2(p[4 * tb], p[4 * tb + 1]), pack_bf16x2(p[4 * tb + 2], p[4 * tb + 3]));
        }
        if (lane < 16) fbuf[i & 1][hl] = f;
      }
      cur = cur == 2 ? 0 : cur + 1;
    }
    // row sums over the four lanes of a head; log2-sum-exp of a run
    l = sum_xor32(sum_xor16(l));
    if (lane < 16) {
      s_l[hl] = l;
      if (NS > 1) a.lse[(int64_t)j * a.R * a.H + hrow0 + hl] = l > 0.f ? m + __log2f(l) : -INFINITY;
    }
    __syncthreads();
    __syncthreads();
  } else {
    // ---------------- value wave v: latent dims 128 v .. 128 v + 127 ----------------
    const int v = wave - 4, hi = lane >> 5, L = lane & 15, q4 = lane >> 4;
    // latent of tile kt, this wave's group: load i fills rows 4 i + lane / 16, physical chunk lane % 16
    auto issue_lat = [&](int kt, uint16_t* st) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        dma16(cache + (int64_t)key_row(kt * DKT + r) * DROW + 128 * v + (((lane & 15) ^ swl(r)) << 3),
              lds_addr(st + v * DGRP + i * 512));
      }
    };
    // transposed reads: 16-lane group q4 reads rows 16 ks + 8 hi + 4 e + L / 4,
    // columns 32 dt + 16 (q4 & 1) + 4 (L % 4) of the group; the lane's k slots are keys 16 ks + 8 hi + 0..7
    const int tx = 2 * (q4 & 1) + ((L >> 1) & 1);
    floatx16 o[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][hb][r] = 0.f;
    if (nt > 0) issue_lat(0, stages);
    if (nt > 1) issue_lat(1, stages + DSTAGE);
    int prev = 2;   // stage of tile i - 1
    for (int i = 0; i <= nt; ++i) {
      wait_tile<8>(i + 1 < nt);
      barrier();
      uint16_t* st = stages + prev * DSTAGE;
      if (i >= 1) {
        const uint16_t* pb = pbuf[(i - 1) & 1];
        const float f0 = fbuf[(i - 1) & 1][lane & 31], f1 = fbuf[(i - 1) & 1][32 + (lane & 31)];
        bf16x8 pf[2][2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int h = 32 * hb + (lane & 31), ch = (2 * ks + hi) ^ ((h >> 2) & 3);
            pf[hb][ks] = *(const bf16x8*)(pb + h * DKT + (ch << 3));
          }
        bf16x8 cf[4][2];
        const uint16_t* sg = st + v * DGRP;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const int r0 = 16 * ks + 8 * hi + (L >> 2), r1 = r0 + 4;
            const v4s lo = read_tr(sg + r0 * 128 + (((4 * dt + tx) ^ swl(r0)) << 3) + 4 * (L & 1));
            const v4s up = read_tr(sg + r1 * 128 + (((4 * dt + tx) ^ swl(r1)) << 3) + 4 * (L & 1));
            cf[dt][ks] = __builtin_bit_cast(bf16x8, (v8s){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
          }
        // every read of this stage's group has returned: refill it with tile i + 2
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (i + 2 < nt) issue_lat(i + 2, st);
        if (__builtin_amdgcn_ballot_w64(f0 != 1.f || f1 != 1.f)) {   // a head's max moved
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              o[dt][0][r] *= f0;
              o[dt][1][r] *= f1;
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) o[dt][hb] = mfma32(cf[dt][ks], pf[hb][ks], o[dt][hb]);
      } else if (i + 2 < nt) {
        issue_lat(2, stages + 2 * DSTAGE);
      }
      prev = prev == 2 ? 0 : prev + 1;
    }
    __syncthreads();   // row sums and maxima of every head are in LDS
    // lane: heads 32 hb + lane % 32, dims 128 v + 32 dt + 8 rg + 4 hi + 0..3; normalised
    // bf16 results to LDS as [64 heads][512 dims], 16-byte chunk c of head h at c ^ (h & 31)
    uint16_t* so = stages;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 32 * hb + (lane & 31);
      const float lh = s_l[h], inv = lh > 0.f ? 1.f / lh : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c = 16 * v + 4 * dt + rg;
          *(uint2*)(so + h * 512 + ((c ^ (h & 31)) << 3) + 4 * hi) =
              make_uint2(pack_bf16x2(o[dt][hb][4 * rg] * inv, o[dt][hb][4 * rg + 1] * inv),
                         pack_bf16x2(o[dt][hb][4 * rg + 2] * inv, o[dt][hb][4 * rg + 3] * inv));
        }
    }
    __syncthreads();
  }
  // every wave: heads 8 p + wave, one 1 KB row per pass
  uint16_t* out = NS == 1 ? (uint16_t*)a.olat + hrow0 * 512 : (uint16_t*)a.part + ((int64_t)j * a.R * a.H + hrow0) * 512;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int h = 8 * p + wave;
    *(uint4*)(out + (int64_t)h * 512 + 8 * lane) = *(const uint4*)(stages + h * 512 + ((lane ^ (h & 31)) << 3));
  }
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
    decode_attn_kernel<true><<<grid, 512, 0, s>>>(a, n_hg);
  } else {
    if (a.rows_per_seq != 0) return hipErrorInvalidValue;
    decode_attn_kernel<false><<<grid, 512, 0, s>>>(a, n_hg);
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
