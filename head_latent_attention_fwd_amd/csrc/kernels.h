// Internal launch interface between the host API (api.cpp) and the kernels.
// Every launcher enqueues on the given stream and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

// C[b][M, N] = A[b][M, K] . W[b]^T. W is [N, K] (K contiguous) unless w_kn, in
// which case it is [K, N] (N contiguous). Rows n >= n_split of W come from W2
// (row n - n_split), which lets one launch cover two stacked weight matrices.
// Epilogues: EPI_ROWMAJOR writes C[m, n] (ldc). EPI_KV_SPLIT treats the
// N = H*256 columns as per-head [k_nope 128 | v 128] and rows m = b*T + t, and
// writes k_nope to C = KN [B, H, Tp, 128] and v transposed to C2 = VT [B, H, 128, Tp].
// EPI_QROPE (bf16 big-tile path, N = H*192): row-major C with RoPE applied to
// columns 128..191 of every 192-wide head (pairs (d, d + 32), position m % T).
// EPI_SWIGLU (bf16 big-tile path): W = gate, W2 = up (same [N, K] shape);
// C[m, n] = silu(A . W^T)[m, n] * (A . W2^T)[m, n] for N = the intermediate width.
enum { EPI_ROWMAJOR = 0, EPI_KV_SPLIT = 1, EPI_QROPE = 2, EPI_SWIGLU = 3 };
struct KvSplit {
  void* vt; int T, Tp, H;
};
struct RopeEpi {
  const float* cos; const float* sin; int T;
};
struct GemmArgs {
  const void* A; int64_t lda; int64_t batch_a;
  const void* W; int64_t ldw; int64_t batch_w;
  const void* W2; int64_t ldw2; int n_split;
  void* C; int64_t ldc; int64_t batch_c; int c_dtype;
  int M, N, K, batch;
  bool w_kn;
  int epi; KvSplit kv; RopeEpi rope;
  // split-K (batch == 1, big-tile path only): part[s][M][N] fp32 partial sums
  // of K chunk s; C is not written
  int k_splits; float* part;
};

// Store of one output element for the EPI_KV_SPLIT layout (m = b*T + t, n = h*256 + j).
template <typename T_>
__device__ __forceinline__ void kv_split_store(const KvSplit& s, T_* kn, T_* vt, int m, int n, T_ v) {
  const int b = m / s.T, t = m - b * s.T, h = n >> 8, j = n & 255;
  const int64_t bh = (int64_t)b * s.H + h;
  if (j < 128) kn[(bh * s.Tp + t) * 128 + j] = v;
  else vt[(bh * 128 + (j - 128)) * s.Tp + t] = v;
}
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);
// Number of K chunks the big-tile path would use for this shape (1 = no split;
// a split is worth it when the output has too few 256x256 tiles to fill the chip).
int gemm_bf16_splits(const GemmArgs& g);
// launch length of g on the big-tile kernels in units of one round of 256 x 256
// tiles on 256 CUs (split: as gemm_bf16_splits would run it)
double gemm_bf16_cost(const GemmArgs& g, bool split);
// whether launch_gemm_bf16 takes g with epi = EPI_QROPE / EPI_SWIGLU
bool gemm_bf16_qrope_ok(const GemmArgs& g);
bool gemm_bf16_swiglu_ok(const GemmArgs& g);
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);

// Block-scaled e4m3 GEMM. W2/w2_scale as in GemmArgs (n_split multiple of 128).
struct GemmFp8Args {
  const uint8_t* A; const float* a_scale;          // [M, K], [M, K/128]
  const uint8_t* W; const float* w_scale;          // [N, K], [ceil(N/128), K/128]
  const uint8_t* W2; const float* w2_scale; int n_split;
  void* C; int64_t ldc; int c_dtype;
  int M, N, K;
  int epi; KvSplit kv; RopeEpi rope;
  // split-K (256x256 path, fp32 row-major output): chunk s of the 128-wide K
  // groups writes its partial sums to (float*)C + s * split_stride
  int k_splits; int64_t split_stride;
};
hipError_t launch_gemm_fp8(const GemmFp8Args& g, hipStream_t s);
// whether launch_gemm_fp8 takes g with epi = EPI_QROPE
bool gemm_fp8_qrope_ok(const GemmFp8Args& g);

// Decode-shaped GEMM (M <= 128): C[z][M, N] = A[z][M, K] . W[z][N, K]^T with
// N tiles of nt (64 or 128) columns and `splits` K chunks of kc (multiple of
// 64; K % 64 == 0). One split: bf16 C. Several: fp32 partials P[split][M][N].
struct SkinnyArgs {
  const void* A; int64_t lda; int64_t batch_a;
  const void* W; int64_t ldw; int64_t batch_w;
  const void* W2; int64_t ldw2; int n_split;
  void* C; int64_t ldc; int64_t batch_c;
  float* P; int64_t ps;   // partial of split s, row m: P + s*ps + m*N
  int M, N, K, kc, batch;
  // e4m3 operands (launch_gemm_skinny_fp8): A codes with 1x128 group scales
  // as[z*batch_as + m*lds + k/128]; W codes with 128x128 block scales
  // ws[z*batch_ws + (n/128)*ldws + k/128] (ws2 for the rows of W2, n - n_split)
  const float* as; int64_t lds; int64_t batch_as;
  const float* ws; const float* ws2; int ldws; int64_t batch_ws;
  // optional e4m3 output instead of C (fp8 kernel, nt = N = 128, one split):
  // row m of batch z -> codes qc[m*ldc + z*batch_c + n], scale qs[m*ldc/128 + z*batch_c/128]
  // of its bf16-rounded values, one 1x128 group per row
  uint8_t* qc; float* qs;
};
hipError_t launch_gemm_skinny(const SkinnyArgs& g, int nt, int splits, hipStream_t s);
// The same product with e4m3 A and W (strides in bytes = elements; K, kc,
// lda, ldw multiples of 128 / 16; n_split a multiple of 128; nt 64 or 128).
hipError_t launch_gemm_skinny_fp8(const SkinnyArgs& g, int nt, int splits, hipStream_t s);
// out[m, n] = sum_s P[s][m][n] as bf16 (row stride ldo).
hipError_t launch_splitk_reduce(const float* P, int S, int M, int N, void* out, int64_t ldo, hipStream_t s);

struct NormRopeArgs {
  const void* in; int64_t ld_in; int in_dtype;
  void* out; int64_t ld_out; int out_dtype;
  int rows, norm_dim; const float* gamma; float eps;
  int rope_off, rope_heads, rope_stride;
  const float* cos_tab; const float* sin_tab; int rope_len;
  const int32_t* pos; int pos_period;
  // optional second copy of the rotated slice (rope_heads == 1): row m = b*T + t
  // goes to kpe[(b*kpe_tp + t)*64], T = pos_period
  void* kpe; int kpe_tp;
  // in_splits > 1: the input is the sum of in_splits fp32 partial arrays
  // split_stride elements apart (split-K GEMM output)
  int in_splits; int64_t split_stride;
};
hipError_t launch_rmsnorm_rope(const NormRopeArgs& a, hipStream_t s);
// Both RMSNorms of a down-projection row [c_q (Dq) | latent (L) | k_pe (64)]
// and the RoPE of k_pe in one pass (bf16 outputs): q_out[m] = norm(c_q),
// kv_out[m] = [norm(latent) | RoPE(k_pe)]. The input is bf16 or the sum of
// in_splits fp32 partial arrays split_stride elements apart (split order).
// kv_pos_stride > 0: the kv row goes to kv_out + m*ld_kv + pos[m]*kv_pos_stride
// and is skipped when pos[m] is outside [0, kv_pos_max) (a cache append).
// Position of row m: pos[m], else m % pos_period. Needs Dq, L, ld_in multiples
// of 4 and (Dq + L + 64) / 4 <= 1024.
struct QkvNormArgs {
  const void* in; int64_t ld_in; int in_dtype; int in_splits; int64_t split_stride;
  int rows, Dq, L;
  const float* gq; const float* gkv; float eps;
  void* q_out; int64_t ld_q;
  // kv entry of row m: with kv_pos_stride > 0 (decode) kv_out + m*ld_kv + pos[m]*kv_pos_stride;
  // else with kv_batch_stride > 0 kv_out + b*kv_batch_stride + (pos_off + t)*ld_kv
  // (m = b*pos_period + t); else kv_out + m*ld_kv
  void* kv_out; int64_t ld_kv; int64_t kv_pos_stride; int kv_pos_max; int64_t kv_batch_stride;
  void* kpe; int kpe_tp;   // optional copy of the rotated k_pe: row m -> kpe[(b*kpe_tp + pos_off + t)*64]
  const float* cos_tab; const float* sin_tab; int rope_len;
  // position of row m: pos[m] if pos is set, else pos_off + m % pos_period
  const int32_t* pos; int pos_period; int pos_off;
  // optional e4m3 copy of the normalised q (Dq % 128 == 0): codes [rows, Dq] and
  // 1x128 scales [rows, Dq/128] of its bf16 values, as launch_quant_1x128 makes them
  uint8_t* q_codes; float* q_scales;
  // the same for the normalised latent (L % 128 == 0): codes [rows, L], scales [rows, L/128]
  uint8_t* kv_codes; float* kv_scales;
  // optional separate source of the 64 k_pe inputs of each row: the sum of kpe_splits (<= 8)
  // fp32 partials kpe_in[s * kpe_split_stride + m * 64 + j] (in split order) instead of
  // the row's last 64 elements of `in`
  const float* kpe_in; int kpe_splits; int64_t kpe_split_stride;
  // e4m3 weights: each latent entry written as its 1x128 e4m3 view (bf16 of code x
  // scale, the value kv_b's quantiser maps it to) instead of the bf16 latent
  bool kv_view;
};
hipError_t launch_qkv_norm(const QkvNormArgs& a, hipStream_t s);
// In place: the first L elements (L % 128 == 0) of each of `rows` bf16 rows, `stride`
// elements apart, replaced by their 1x128 e4m3 view.
hipError_t launch_latent_e4m3_view(void* cache, int64_t rows, int64_t stride, int L, hipStream_t s);
hipError_t launch_rope_table(float* c, float* sn, int n_pos, float base, hipStream_t s);
hipError_t launch_quant_1x128(const void* a, int64_t lda, int a_dtype, int M, int K,
                              uint8_t* q, float* scales, hipStream_t s);
hipError_t launch_quant_block128(const float* w, int N, int K, uint8_t* q, float* scales, hipStream_t s);
// dst[r*dld + c] = src[r*sld + c] for r < rows, c < cols (16-bit elements;
// cols, sld, dld multiples of 8 and both pointers 16-byte aligned).
hipError_t launch_copy_rows(const uint16_t* src, int64_t sld, uint16_t* dst, int64_t dld, int64_t rows, int cols,
                            hipStream_t s);
// dst[z][c][r] = src[z][r][c] (16-bit elements) for r < rows, c < cols; row
// strides sld / dld, batch strides sb / db.
hipError_t launch_transpose16(const uint16_t* src, int64_t sld, int64_t sb, uint16_t* dst, int64_t dld, int64_t db,
                              int rows, int cols, int batch, hipStream_t s);
// Row r of gu [rows, ld] holds gate in columns [0, cols) and up in [cols, 2 cols)
// (bf16, or with nsplit > 0 the fp32 split-K partials gu + s*split_stride,
// summed in split order): h = bf16(silu(gate) * up), quantised in 1x128 groups
// to codes hq [rows, cols] and scales hs [rows, cols/128] (cols % 128 == 0,
// ld % 8 == 0, 16-byte aligned).
hipError_t launch_silu_mul_quant(const void* gu, int64_t ld, int nsplit, int64_t split_stride, int rows, int cols,
                                 uint8_t* hq, float* hs, hipStream_t s);
// h[i] = silu(g[i]) * u[i] over n bf16 values (n % 8 == 0, 16-byte aligned).
hipError_t launch_silu_mul(const void* g, const void* u, void* h, int64_t n, hipStream_t s);
// mask [B, T, ceil(Tk/32)]: bit t of row (b, s) is set iff t appears in
// idx[b, s, :] and t <= P + s (query s sits at position P + s) and t < Tk.
hipError_t launch_topk_bitmask(const int32_t* idx, int B, int T, int k, int P, int Tk, uint32_t* mask, hipStream_t s);
// Copies the rotated shared keys of cache rows [0, P) ([B, cache_ld] per
// sequence, k_pe at element offset kpe_off of each row_ld-wide row) into kpe [B, Tp, 64].
hipError_t launch_gather_kpe(const void* cache, int64_t cache_ld, int row_ld, int kpe_off, int B, int P, void* kpe,
                             int Tp, hipStream_t s);

// Prefill attention. T queries per sequence at positions P..P+T-1 over the
// Tk = P + T keys 0..P+T-1 (P = 0: empty cache). q [B*T, H*192] (rope
// applied), kn [B, H, Tp, 128], vt [B, H, 128, Tp], kpe [B, Tp, 64] (rotated
// shared key), optional bitmask [B, T, ceil(Tk/32)], out [B*T, H*128].
// Tp = Tk rounded up to 64; the padding keys (t >= Tk) of kn, vt and kpe must
// hold finite values.
struct PrefillAttnArgs {
  const void* q; const void* kn; const void* vt; const void* kpe;
  const uint32_t* mask; void* out;
  int B, T, Tp, H; float scale; int P;
  // optional (bf16 kernel): the output as e4m3 codes [B*T, H*128] with one 1x128
  // scale per (row, head) [B*T, H], quantised from its bf16 values, instead of out
  uint8_t* oq; float* os;
};
// Zeroes the padding keys t in [T, Tp) of kn, vt and kpe (no-op when T == Tp).
hipError_t launch_zero_kv_padding(void* kn, void* vt, void* kpe, int B, int H, int T, int Tp, int elem_bytes,
                                  hipStream_t s);
hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, hipStream_t s);
hipError_t launch_prefill_attn_f32(const PrefillAttnArgs& a, hipStream_t s);

// Decode pieces.
constexpr int DECODE_TOPK_MAX = 2048;
constexpr int DECODE_MAX_SPLITS = 16;
// Latent-space attention, one query row q at a time over cache rows C_t =
// [latent 512 | rope 64] (bf16): o_lat[q, h] = sum_t softmax_t(scale * q_lat[q, h] . C_t) C_t[:512].
struct DecodeAttnArgs {
  const void* qlat;      // [R, H, 576] bf16: absorbed query (512) | rotated q_pe (64)
  const void* cache;     // [S, max_len, 576] bf16
  const int32_t* cache_len;   // decode: row q is sequence q with last key cache_len[q]
  int R, H, max_len; float scale;
  // rows_per_seq > 0 (selected keys only): row q is token q % rows_per_seq of
  // sequence q / rows_per_seq, its last key that position (absorbed prefill)
  int rows_per_seq;
  // Selected keys (optional): the compacted lists launch_decode_compact makes,
  // row q's live positions keys[q*kstride .. + nkeys[q]) (ascending, distinct)
  const int32_t* keys; const int32_t* nkeys; int kstride;
  // The row's keys are cut into `splits` runs of whole 32-key tiles. splits == 1:
  // olat [R, H, 512] bf16 is the normalised output. splits > 1: part
  // [splits][R*H][512] bf16 holds each run's normalised output and lse
  // [splits][R*H] its log2-sum-exp of the scaled scores (-inf for an empty run).
  int splits;
  void* olat; void* part; float* lse;
};
hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s);
// Splits that fill the chip for `rows` query rows of H heads over at most
// max_keys keys (at most DECODE_MAX_SPLITS, about four tiles or more each).
int decode_splits(int rows, int H, int max_keys);
// keys[q*kstride ..] = row q's listed positions t with 0 <= t <= last(q) (last(q) =
// q % rows_per_seq when rows_per_seq > 0, else cache_len[q]; rows with
// last(q) outside [0, max_len) get none), ascending, repeats removed;
// nkeys[q] = their number. idx [rows, topk] with topk <= DECODE_TOPK_MAX; kstride >= topk.
hipError_t launch_decode_compact(const int32_t* idx, int topk, const int32_t* cache_len, int rows_per_seq, int rows,
                                 int max_len, int32_t* keys, int kstride, int32_t* nkeys, hipStream_t s);
// olat[r] from the split partials of launch_decode_attn, merged in split order (rows = R*H).
hipError_t launch_decode_combine(const void* part, const float* lse, int splits, int64_t rows, void* olat,
                                 hipStream_t s);
// o[b, 128 h + j] = sum_c W_UV_h[j, c] o_lat[b, h, c] (W_UV_h = wkv_b rows [256h + 128, 256h + 256),
// kv_lora_rank 512), o_lat merged from the attention's split partials (splits == 1: part = o_lat).
struct UnabsorbArgs {
  const void* part; const float* lse; int splits;   // as DecodeAttnArgs (rows B*H)
  const void* wkv_b; const float* w_scale;          // bf16, or e4m3 codes with block scales [2H, 4]
  void* o; int64_t ldo;                             // o [B, ldo] bf16 (ldo = H*128), or NULL
  uint8_t* oq; float* os;                           // or/and e4m3 codes [B, ldo] + scales [B, ldo/128]
  int B, H;
};
hipError_t launch_decode_unabsorb(const UnabsorbArgs& a, hipStream_t s);
// Size of the library-held scratch of the allocation-free decode attention,
// and its device address on the current device (looked up once per device).
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);
// q_lat[b, h] = [q_nope[b, h] . W_UK_h | RoPE(q_pe[b, h], cache_len[b])] for kv_lora_rank 512;
// q [B, H*192], wkv_b [H*256, 512] (bf16, or e4m3 codes with block scales
// w_scale [2H, 4]; w_scale == nullptr for bf16), qlat [B, H, 576].
hipError_t launch_decode_absorb(const void* q, const void* wkv_b, const float* w_scale, void* qlat,
                                const int32_t* cache_len, const float* cos_tab, const float* sin_tab, int B, int H,
                                int max_len, hipStream_t s);

}  // namespace mla
