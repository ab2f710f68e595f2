/*
 * mla.h — C ABI of the MI355X (gfx950) multi-head latent attention forward.
 *
 * What is computed follows the model-atlas pages on MLA:
 *   "Kimi K2 · Query compression"            (query path, module init, parameter table)
 *   "Kimi K2 · Output projection"            (Delta_attn = o W_O, [out, in] weights)
 *   "Kimi K2 · Down projection"              (FP8 e4m3, 128 x 128 weight blocks, dynamic activations)
 *   "DeepSeek-V3.2-Exp · Sparse attention"   (prefill: scores, top-k + causal mask, softmax, PV)
 *   "DeepSeek-V3.2-Exp · Output projection"  (decode at p = 1000; softmax_scale from the MLA init)
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *    allocates device memory; scratch comes from a caller workspace whose size
 *    the *_workspace_size queries return (mla_decode_attention_noalloc instead
 *    uses a fixed scratch array the library holds per GPU). Host-side structs
 *    are read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued asynchronously on it; no entry point synchronises.
 *  - Matrices are row-major. Weights are [out, in] (K contiguous). Activations
 *    are [rows, features] with rows = B*T and per-head features packed head-major.
 *  - bf16 = bfloat16 storage, fp32 accumulation. e4m3 = OCP FP8 E4M3FN bytes.
 *  - Return value: an mla_status. On failure nothing has been enqueued, except
 *    MLA_HIP_ERROR from a launch, after which the stream's contents are
 *    unspecified. mla_last_error() gives a thread-local message.
 *  - Results are deterministic: no atomics in reductions, fixed split counts.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_INVALID_ARG = 1,   /* null pointer, bad or inconsistent size, workspace too small */
  MLA_UNSUPPORTED = 2,   /* valid but not built: head dims other than 128/64/128, K % 128 != 0 for fp8, ... */
  MLA_HIP_ERROR = 3      /* a HIP launch or query failed */
} mla_status;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_E4M3 = 2
} mla_dtype;

/* MLA sizes (DeepSeek-V3.2-Exp · Output projection, "Code": the MLA init names
 * dim, q_lora_rank, kv_lora_rank, n_heads and the three head dims). The build
 * supports qk_nope_head_dim = 128, qk_rope_head_dim = 64, v_head_dim = 128.
 * softmax_scale is normally (qk_nope + qk_rope)^-0.5; rms_eps is the RMSNorm
 * epsilon (inside the square root). */
typedef struct {
  int32_t dim;
  int32_t q_lora_rank;
  int32_t kv_lora_rank;
  int32_t n_heads;
  int32_t qk_nope_head_dim;
  int32_t qk_rope_head_dim;
  int32_t v_head_dim;
  float softmax_scale;
  float rms_eps;
} mla_dims;

/* Device pointers to the MLA weights (Kimi K2 · Query compression, "Code":
 * module init). All projections are bias-free, [out, in]:
 *   wq_a  [q_lora_rank, dim]                    q_norm_w  [q_lora_rank]  fp32
 *   wq_b  [n_heads*192, q_lora_rank]             per head: 128 non-rotated, then 64 rotated
 *   wkv_a [kv_lora_rank + 64, dim]               latent first, then the shared rotary key
 *   kv_norm_w [kv_lora_rank] fp32
 *   wkv_b [n_heads*256, kv_lora_rank]            per head: 128 key (non-rotated), then 128 value
 *   wo    [dim, n_heads*128]
 * weight_dtype is MLA_F32, MLA_BF16 or MLA_E4M3. With MLA_E4M3 every *_scale
 * pointer is required: fp32 [ceil(out/128), in/128], one scale per 128 x 128
 * block (Kimi K2 · Down projection, quantization_config); otherwise they are
 * ignored. */
typedef struct {
  int32_t weight_dtype;
  const void* wq_a;  const float* wq_a_scale;
  const float* q_norm_w;
  const void* wq_b;  const float* wq_b_scale;
  const void* wkv_a; const float* wkv_a_scale;
  const float* kv_norm_w;
  const void* wkv_b; const float* wkv_b_scale;
  const void* wo;    const float* wo_scale;
} mla_weights;

MLA_API const char* mla_version(void);
/* Message of the last failed call on this thread ("" if none). */
MLA_API const char* mla_last_error(void);

/* ------------------------------------------------------------------------
 * Whole-path entry points
 * ------------------------------------------------------------------------ */

/* Bytes of workspace mla_prefill needs for these sizes (0 on invalid input). */
MLA_API size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t act_dtype,
                                  int32_t B, int32_t T, int32_t topk);

/* MLA prefill with an empty cache (DeepSeek-V3.2-Exp · Sparse attention, mode
 * prefill: the path taken for more than one position; Kimi K2 · Output
 * projection for the head flatten and o_proj). Positions are 0..T-1.
 *   x        [B, T, dim]   act_dtype (MLA_F32 with F32 weights, or MLA_BF16)
 *   rope_cos, rope_sin  fp32 [rope_len, 32]: cos/sin of pos * 10000^(-d/32)
 *            for pos = row (see mla_rope_table); rope_len >= T
 *   topk_idx [B, T, topk] int32 or NULL. Key t is live for query s iff t <= s
 *            and (topk_idx == NULL or t appears in row (b, s)); -1 pads. Every
 *            query must keep at least one live key (its own position suffices).
 *   out      [B, T, dim]   act_dtype
 *   kv_cache_out [B, T, kv_lora_rank + 64] bf16 (fp32 for MLA_F32) or NULL:
 *            receives the per-position [normalised latent | rotated k_pe];
 *            with e4m3 weights the latent in its 1x128 e4m3 view (see
 *            mla_latent_e4m3_view), the form kv_b's quantiser gives it.
 *   ws, ws_bytes  workspace of at least mla_prefill_workspace_size(...) bytes,
 *            256-byte aligned. */
MLA_API int mla_prefill(const mla_dims* dims, const mla_weights* w, const void* x, int32_t act_dtype,
                int32_t B, int32_t T, const float* rope_cos, const float* rope_sin, int32_t rope_len,
                const int32_t* topk_idx, int32_t topk, void* out, void* kv_cache_out,
                void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace mla_prefill_cached needs (0 on invalid input). */
MLA_API size_t mla_prefill_cached_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t B, int32_t T,
                                         int32_t start_pos, int32_t topk);

/* MLA prefill of a chunk of T new tokens per sequence after start_pos cached
 * ones (chunked prefill). The pages define prefill with an empty cache
 * (DeepSeek-V3.2-Exp · Sparse attention, mode prefill) and the cache as the
 * per-position [normalised latent | rotated k_pe] that decode scores
 * (Explanation there); this entry point reads them together: token s of the
 * chunk sits at position start_pos + s, its entry is written to
 * kv_cache[b, start_pos + s], and it attends keys 0..start_pos+s, the cached
 * ones up-projected by kv_b exactly like the chunk's own. With start_pos = 0
 * the result is mla_prefill's; chaining chunks gives the rows of one prefill
 * over their concatenation.
 *   x         [B, T, dim] bf16
 *   kv_cache  [B, max_len, kv_lora_rank + 64] bf16, in/out: rows [0, start_pos)
 *             are read, rows [start_pos, start_pos + T) are written; 16-byte aligned
 *   start_pos >= 0, start_pos + T <= max_len (same for every sequence)
 *   rope_cos, rope_sin  fp32 [rope_len, 32], rope_len >= start_pos + T
 *   topk_idx  [B, T, topk] int32 or NULL: absolute key positions; key t is live
 *             for chunk row s iff t <= start_pos + s and (no topk_idx or t is
 *             listed in row (b, s)); -1 pads
 *   out       [B, T, dim] bf16
 * Weights bf16 or e4m3 (block-scaled, as for mla_prefill; the chunk's entries
 * are then written in their e4m3 view, and cached latents in either form give
 * the same result, since kv_b quantises them). */
MLA_API int mla_prefill_cached(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B, int32_t T,
                       int32_t start_pos, void* kv_cache, int32_t max_len, const float* rope_cos,
                       const float* rope_sin, int32_t rope_len, const int32_t* topk_idx, int32_t topk, void* out,
                       void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace mla_decode and mla_decode_sparse need for bf16 or e4m3
 * weights (0 on invalid input). */
MLA_API size_t mla_decode_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t B, int32_t max_len);

/* Single-token MLA decode, latent-absorbed (DeepSeek-V3.2-Exp · Sparse
 * attention, "Explanation": a single decoded token scores the cached latent
 * directly; DeepSeek-V3.2-Exp · Output projection at p = 1000).
 * Per sequence b with P = cache_len[b]: the new token at position P produces
 * its cache entry [normalised latent | rotated k_pe], which is written to
 * kv_cache[b, P]; it then attends slots 0..P with kv_b's key half folded into
 * the query and its value half applied after the attention, then wo.
 *   x         [B, dim] bf16
 *   kv_cache  [B, max_len, kv_lora_rank + 64] bf16, in/out (only slot P of
 *             each sequence is written)
 *   cache_len [B] int32 DEVICE array, 0 <= cache_len[b] < max_len (checked on
 *             the device: an out-of-range sequence is skipped and its output
 *             row is set to zero)
 *   max_len   <= 2^20 (MLA_INVALID_ARG otherwise)
 *   rope_cos, rope_sin  fp32 [rope_len, 32], rope_len >= max_len
 *   out       [B, dim] bf16
 * Weights bf16, or e4m3 with 128x128 block scales (Kimi K2 · Down projection,
 * quantization_config: e4m3, dynamic activation scheme, 128x128 weight
 * blocks). With e4m3 every Linear is applied as prefill applies it: the
 * inputs of q_a|kv_a, q_b and wo are quantised in dynamic 1x128 groups, and
 * kv_b acts on each cached latent quantised in 1x128 groups; the absorbed
 * form reaches that result with the dequantised W_UK and W_UV and each
 * latent's dequantised 1x128 value. With e4m3 weights the cache holds every
 * latent in that dequantised form (its e4m3 view, as mla_prefill,
 * mla_prefill_cached and mla_decode write it with e4m3 weights, or as
 * mla_latent_e4m3_view converts a cache of plain latents): the new entry is
 * written so, and cached latents are read as they are. Needs kv_lora_rank = 512, n_heads a
 * multiple of 64, dim and q_lora_rank multiples of 128 for e4m3, and 16-byte
 * aligned x, out, cache and norm weights (MLA_UNSUPPORTED otherwise). The
 * key range of each sequence may be cut into several runs whose partial
 * results are merged in a fixed order, so results are deterministic. */
MLA_API int mla_decode(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B,
               void* kv_cache, int32_t max_len, const int32_t* cache_len,
               const float* rope_cos, const float* rope_sin, int32_t rope_len,
               void* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Building blocks (each is also a step of the paths above)
 * ------------------------------------------------------------------------ */

/* C[M, N] = A[M, K] . W[N, K]^T (a bias-free Linear with [out, in] weights,
 * Kimi K2 · Output projection formula). A, W bf16; C bf16 or fp32 (c_dtype).
 * Leading dims in elements; K % 8 == 0, lda/ldw % 8 == 0, A/W 16-byte aligned. */
MLA_API int gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
              int32_t c_dtype, int32_t M, int32_t N, int32_t K, void* stream);

/* Same product in fp32 (A, W, C fp32), for the fp32 path. */
MLA_API int gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, float* C, int64_t ldc,
             int32_t M, int32_t N, int32_t K, void* stream);

/* Block-scaled FP8 product (Kimi K2 · Down projection, quantization_config):
 *   C[m, n] = sum_g a_scale[m, g] * w_scale[n / 128, g] * sum_{k in g} Aq[m, k] * Wq[n, k]
 * over 128-wide groups g along K. Aq [M, K] e4m3 with a_scale fp32 [M, K/128];
 * Wq [N, K] e4m3 with w_scale fp32 [ceil(N/128), K/128]; all contiguous.
 * C [M, N] (ldc) bf16 or fp32. K % 128 == 0. */
MLA_API int gemm_fp8_blockscaled(const uint8_t* Aq, const float* a_scale, const uint8_t* Wq, const float* w_scale,
                         void* C, int64_t ldc, int32_t c_dtype, int32_t M, int32_t N, int32_t K, void* stream);

/* Decode-shaped products: the same bias-free Linear for a batch of single
 * tokens, M <= 128 rows (DeepSeek-V3.2-Exp · Output projection, decode at
 * p = 1000: [B, 1, 16384] -> [B, 1, 7168]). Every weight byte is streamed once
 * from HBM; a long K is cut into chunks whose fp32 partials (in the
 * workspace) are summed in a fixed order. These are the kernels mla_decode
 * runs for q_a|kv_a, q_b and wo.
 *   gemm_bf16_decode: A [M, K], W [N, K] bf16, C [M, N] bf16; K % 64 == 0
 *   gemm_fp8_decode:  Aq [M, K] e4m3 codes with a_scale [M, K/128], Wq [N, K]
 *                     with w_scale [ceil(N/128), K/128] (block-scaled product
 *                     as gemm_fp8_blockscaled), C [M, N] bf16; K % 128 == 0
 * All contiguous and 16-byte aligned; ws of gemm_decode_workspace_size bytes,
 * 256-byte aligned. */
MLA_API size_t gemm_decode_workspace_size(int32_t weight_dtype, int32_t M, int32_t N, int32_t K);
MLA_API int gemm_bf16_decode(const void* A, const void* W, void* C, int32_t M, int32_t N, int32_t K, void* ws,
                             size_t ws_bytes, void* stream);
MLA_API int gemm_fp8_decode(const uint8_t* Aq, const float* a_scale, const uint8_t* Wq, const float* w_scale,
                            void* C, int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, void* stream);

/* Row-wise RMSNorm and RoPE (the q_a / kv_a layernorms and the rotary part of
 * the query and of the shared key; Kimi K2 · Query compression, "Code").
 * For each of `rows` rows:
 *   if norm_dim > 0: out[:norm_dim] = gamma * in[:norm_dim] / sqrt(mean(in[:norm_dim]^2) + eps)
 *   for h < rope_heads: the 64 values at rope_off + h*rope_stride are rotated
 *     rotate-half style (dim d pairs with d+32) by cos/sin row pos(row), where
 *     pos(row) = pos ? pos[row] : row % pos_period.
 * Other elements of `out` are not written. in == out is allowed.
 * in_dtype/out_dtype: MLA_F32 or MLA_BF16; math in fp32. gamma fp32 (may be
 * NULL when norm_dim == 0). */
MLA_API int rmsnorm_rope(const void* in, int64_t ld_in, int32_t in_dtype, int32_t rows, int32_t norm_dim,
                 const float* gamma, float eps, int32_t rope_off, int32_t rope_heads, int32_t rope_stride,
                 const float* cos_tab, const float* sin_tab, int32_t rope_len, const int32_t* pos,
                 int32_t pos_period, void* out, int64_t ld_out, int32_t out_dtype, void* stream);

/* The fused prefill attention step alone (DeepSeek-V3.2-Exp · Sparse attention,
 * "Code": scores over [non-rotated | shared rotary] keys, selection + causal
 * mask, softmax, weighted values), never materialising the T x T scores.
 * With Tp = T rounded up to a multiple of 64:
 *   q      [B*T, H*192]    per head [q_nope 128 | q_pe 64], RoPE already applied
 *   k_nope [B, H, Tp, 128] per-head non-rotated keys (kv_b output, key half)
 *   v_t    [B, H, 128, Tp] per-head values, transposed (kv_b output, value half)
 *   k_pe   [B, Tp, 64]     rotated shared key
 *   mask   [B, T, ceil(T/32)] uint32 selection bits (mla_topk_to_bitmask) or NULL
 *          for causal only; a key is live iff its bit is set and t <= s
 *   out    [B*T, H*128]
 * The padding keys t in [T, Tp) of k_nope, v_t and k_pe are overwritten with 0.
 * dtype MLA_BF16 or MLA_F32 for every tensor. Rows with no live key give 0. */
MLA_API int mla_prefill_attention(const void* q, const void* k_nope, const void* v_t, const void* k_pe,
                                  const uint32_t* mask, void* out, int32_t dtype, int32_t B, int32_t T,
                                  int32_t H, float scale, void* stream);

/* Bytes of workspace mla_decode_attention needs (0 on invalid input): the
 * per-run partial outputs when the key range of a sequence is cut into runs. */
MLA_API size_t mla_decode_attention_workspace_size(int32_t B, int32_t H, int32_t max_len);

/* The absorbed decode attention step alone (DeepSeek-V3.2-Exp · Sparse
 * attention, "Explanation"): for each sequence b and head h,
 *   o_lat[b, h] = sum_{t <= cache_len[b]} softmax_t(scale * q_lat[b, h] . C[b, t]) C[b, t, :512]
 *   q_lat [B, H, 576] bf16 (latent-space query 512 | rotated q_pe 64)
 *   cache [B, max_len, 576] bf16; cache_len [B] int32 device array; max_len <= 2^20
 *   o_lat [B, H, 512] bf16 (zero for sequences whose cache_len is out of range)
 *   ws, ws_bytes  workspace of at least mla_decode_attention_workspace_size(B, H,
 *   max_len) bytes, 256-byte aligned (partial results of the key runs, merged
 *   in a fixed order)
 * H must be a multiple of 64; q_lat, cache and o_lat 16-byte aligned. */
MLA_API int mla_decode_attention(const void* q_lat, const void* cache, const int32_t* cache_len, void* o_lat,
                                 int32_t B, int32_t H, int32_t max_len, float scale, void* ws, size_t ws_bytes,
                                 void* stream);

/* The same decode attention for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the partial results of the key runs live in a 32 MiB
 * scratch array the library holds on each GPU it runs on (kept until the
 * process ends). Arguments and result as mla_decode_attention; sizes whose
 * workspace (mla_decode_attention_workspace_size) exceeds 32 MiB are
 * rejected with MLA_INVALID_ARG. Calls on one GPU share that array: calls
 * that overlap on one GPU (other streams, other host threads) race and must
 * be ordered by the caller. Allocates no memory. */
MLA_API int mla_decode_attention_noalloc(const void* q_lat, const void* cache, const int32_t* cache_len,
                                         void* o_lat, int32_t B, int32_t H, int32_t max_len, float scale,
                                         void* stream);

/* e4m3 view of cached latents, in place (Kimi K2 · Down projection,
 * quantization_config: kv_b is an e4m3 Linear whose input is quantised in
 * dynamic 1x128 groups): the first kv_lora_rank bf16 elements of each of `rows`
 * rows, row_stride elements apart, are replaced by the value their quantisation
 * stands for, bf16(code x s) with s = amax / 448 and codes as in
 * mla_quant_e4m3_1x128. The view is a fixed point of that quantisation, so kv_b
 * gives the same product on it as on the plain latent; it is the cache form the
 * e4m3 calls write and mla_decode reads. kv_lora_rank % 128 == 0, row_stride %
 * 8 == 0 and a 16-byte aligned cache (MLA_UNSUPPORTED otherwise). */
MLA_API int mla_latent_e4m3_view(void* cache, int64_t rows, int64_t row_stride, int32_t kv_lora_rank,
                                 void* stream);

/* cos/sin table for RoPE: cos_tab[p, d] = cos(p * base^(-d/32)), sin likewise,
 * for p < n_pos, d < 32, evaluated in fp64 and stored fp32. */
MLA_API int mla_rope_table(float* cos_tab, float* sin_tab, int32_t n_pos, float base, void* stream);

/* Dynamic activation quantisation to e4m3, one fp32 scale per row and per 128
 * elements along K (Kimi K2 · Down projection: activation_scheme dynamic):
 *   s = amax(group) / 448 (fp32; 0 for an all-zero group), q = e4m3_rne(a / s)
 * with the quotient in fp32. a: [M, K] (lda) MLA_F32 or MLA_BF16; q [M, K]
 * contiguous; scales [M, K/128]. K % 128 == 0, lda % 8 == 0, a and q 16-byte
 * aligned (MLA_UNSUPPORTED otherwise). */
MLA_API int mla_quant_e4m3_1x128(const void* a, int64_t lda, int32_t a_dtype, int32_t M, int32_t K,
                         uint8_t* q, float* scales, void* stream);

/* Weight quantisation to e4m3 with one fp32 scale per 128 x 128 block of
 * [N, K] (Kimi K2 · Down projection, quantization_config weight_block_size).
 * s = amax(block)/448 over the valid elements, q = e4m3_rne(w / s) with the
 * quotient in fp32. w fp32 [N, K]; q [N, K]; scales [ceil(N/128), ceil(K/128)]. */
MLA_API int mla_quant_e4m3_block128(const float* w, int32_t N, int32_t K, uint8_t* q, float* scales, void* stream);

/* Top-k selection + causal mask as bits (DeepSeek-V3.2-Exp · Sparse
 * attention, "Code" and the M^sel input): mask[b, s, w] bit j is 1 iff key
 * t = 32w + j appears in topk_idx[b, s, :] and t <= s. topk_idx [B, T, topk]
 * int32 (-1 and out-of-range entries ignored); mask uint32 [B, T, ceil(T/32)]. */
MLA_API int mla_topk_to_bitmask(const int32_t* topk_idx, int32_t B, int32_t T, int32_t topk,
                        uint32_t* mask, void* stream);

/* Single-token decode over selected cache positions (DeepSeek-V3.2-Exp ·
 * Sparse attention: the indexer's selection, applied with the causal mask, in
 * the latent form a decoded token uses). As mla_decode, except that sequence b
 * attends only the positions listed in topk_idx[b, 0:topk] that are <= its new
 * position cache_len[b] (the new token's own slot must be listed to be
 * attended).
 *   topk_idx [B, topk] int32 DEVICE array of positions, -1 pads; entries
 *            outside [0, cache_len[b]] are ignored and a repeated position
 *            counts once (the selection is a set, as a 0 / -inf mask makes it),
 *            in any order
 *   1 <= topk <= 2048 (MLA_UNSUPPORTED otherwise). Workspace as mla_decode. */
MLA_API int mla_decode_sparse(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B,
                      void* kv_cache, int32_t max_len, const int32_t* cache_len, const int32_t* topk_idx,
                      int32_t topk, const float* rope_cos, const float* rope_sin, int32_t rope_len,
                      void* out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace mla_prefill_absorbed needs (0 on invalid input). */
MLA_API size_t mla_prefill_absorbed_workspace_size(const mla_dims* dims, int32_t B, int32_t T, int32_t topk);

/* Prefill with a top-k selection computed in the absorbed latent form
 * (DeepSeek-V3.2-Exp · Sparse attention: the same scores, selection and causal
 * mask as mla_prefill with topk_idx; the Explanation's latent scoring applied to
 * every token): kv_b's key half is folded into each token's query, every token
 * gathers only its selected cache entries [normalised latent | rotated k_pe]
 * (all heads share them), and the value half is applied after the attention.
 * The work per token is proportional to topk instead of its position.
 *   x [B, T, dim] bf16 (16-byte aligned), bf16 weights, kv_lora_rank = 512, n_heads a multiple of 64
 *   topk_idx [B, T, topk] int32 DEVICE array (required), -1 pads, any order;
 *            key t is live for query s iff t <= s and t is listed (a repeated
 *            position counts once); 1 <= topk <= 2048
 *   out [B, T, dim] bf16; kv_cache_out [B, T, kv_lora_rank + 64] bf16 or NULL
 * Workspace: mla_prefill_absorbed_workspace_size(dims, B, T, topk) bytes, 256-byte aligned. */
MLA_API int mla_prefill_absorbed(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B, int32_t T,
                         const float* rope_cos, const float* rope_sin, int32_t rope_len,
                         const int32_t* topk_idx, int32_t topk, void* out, void* kv_cache_out, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Shared-expert MLP
 * ------------------------------------------------------------------------ */

/* Bytes of workspace mla_swiglu_mlp needs (0 on invalid input). */
MLA_API size_t mla_swiglu_workspace_size(int32_t M, int32_t inter);

/* Shared-expert SwiGLU MLP (Kimi K2 · Down projection: the shared expert
 * applies down_proj to act_fn(gate_proj(x)) * up_proj(x), act_fn = silu,
 * bias-free Linears):
 *   out = (silu(x . Wg^T) * (x . Wu^T)) . Wd^T,  silu(z) = z / (1 + exp(-z))
 *   x [M, hidden] bf16; w_gate, w_up [inter, hidden] bf16; w_down [hidden, inter]
 *   bf16; out [M, hidden] bf16; ws: workspace of mla_swiglu_workspace_size(M,
 *   inter) bytes, 256-byte aligned. hidden and inter multiples of 64, all
 *   pointers 16-byte aligned (MLA_UNSUPPORTED otherwise). The gate / up
 *   products are rounded to bf16 before silu and the product. */
MLA_API int mla_swiglu_mlp(const void* x, int32_t M, int32_t hidden, int32_t inter, const void* w_gate,
                   const void* w_up, const void* w_down, void* out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace mla_swiglu_mlp_e4m3 needs (0 on invalid input). */
MLA_API size_t mla_swiglu_e4m3_workspace_size(int32_t M, int32_t hidden, int32_t inter);

/* The shared-expert SwiGLU MLP with e4m3 weights in the checkpoint's format
 * (Kimi K2 · Down projection, quantization_config: e4m3, dynamic activation
 * scheme, 128x128 weight blocks): every Linear quantises its bf16 input in
 * dynamic 1x128 groups and runs the block-scaled e4m3 product.
 *   w_gate, w_up [inter, hidden] e4m3 codes with scales [inter/128, hidden/128]
 *   fp32; w_down [hidden, inter] codes with scales [hidden/128, inter/128];
 *   x, out [M, hidden] bf16; hidden and inter multiples of 128. The gate and up
 *   products and h are rounded to bf16, as in mla_swiglu_mlp. */
MLA_API int mla_swiglu_mlp_e4m3(const void* x, int32_t M, int32_t hidden, int32_t inter, const void* w_gate,
                        const float* gate_scale, const void* w_up, const float* up_scale,
                        const void* w_down, const float* down_scale, void* out, void* ws, size_t ws_bytes,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
