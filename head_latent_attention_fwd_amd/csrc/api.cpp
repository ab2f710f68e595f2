// Host side of the C ABI declared in include/mla.h: argument checks,
// workspace carving and the launch sequences of the prefill and decode paths.
// Nothing here computes; every step is a kernel enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mla.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}
#define LAUNCH(expr, what)                           \
  do {                                               \
    int rc_ = hip_check((expr), what);               \
    if (rc_ != MLA_OK) return rc_;                   \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base((char*)p) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  }
};

int check_dims(const mla_dims* d) {
  if (!d) return fail(MLA_INVALID_ARG, "dims is NULL");
  if (d->dim <= 0 || d->q_lora_rank <= 0 || d->kv_lora_rank <= 0 || d->n_heads <= 0)
    return fail(MLA_INVALID_ARG, "dims must be positive");
  if (d->qk_nope_head_dim != 128 || d->qk_rope_head_dim != 64 || d->v_head_dim != 128)
    return fail(MLA_UNSUPPORTED, "head dims must be 128/64/128 (got %d/%d/%d)", d->qk_nope_head_dim,
                d->qk_rope_head_dim, d->v_head_dim);
  if (d->dim % 8 || d->q_lora_rank % 8 || d->kv_lora_rank % 8)
    return fail(MLA_UNSUPPORTED, "dim, q_lora_rank and kv_lora_rank must be multiples of 8");
  if (!(d->softmax_scale > 0.f) || !(d->rms_eps >= 0.f)) return fail(MLA_INVALID_ARG, "bad softmax_scale/rms_eps");
  return MLA_OK;
}

int check_weights(const mla_weights* w, int wdt) {
  if (!w) return fail(MLA_INVALID_ARG, "weights is NULL");
  if (w->weight_dtype != wdt) return fail(MLA_INVALID_ARG, "weights->weight_dtype mismatch");
  if (!w->wq_a || !w->q_norm_w || !w->wq_b || !w->wkv_a || !w->kv_norm_w || !w->wkv_b || !w->wo)
    return fail(MLA_INVALID_ARG, "a weight pointer is NULL");
  if (wdt == MLA_E4M3 && (!w->wq_a_scale || !w->wq_b_scale || !w->wkv_a_scale || !w->wkv_b_scale || !w->wo_scale))
    return fail(MLA_INVALID_ARG, "e4m3 weights need every block-scale pointer");
  return MLA_OK;
}

struct PrefillWs {
  void *cqkv, *cqn, *kvc, *q, *kn, *vt, *kpe, *attn, *mask, *aq, *as;
  float* part;      // split-K partials of the joint down-projection (or NULL)
  int qkv_splits;
  float* kpe_part;  // e4m3: split-K partials of the k_pe columns [kpe_splits][M][64] (or NULL)
  int kpe_splits;
};

int pad64(int T) { return (T + 63) & ~63; }

// Longest cache a sequence may have: the attention kernels address a
// sequence's rows through one raw buffer of max_len * 576 bf16 values, whose
// byte size must stay below 2^31.
constexpr int MAX_CACHE_LEN = 1 << 20;

mla::GemmArgs gemm_args(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int cdt, int M,
                        int N, int K);

// Arguments of the joint down-projection [c_q | latent | k_pe] = x . [Wq_a ; Wkv_a]^T.
mla::GemmArgs qkv_args(const mla_dims* d, int adt, const void* x, const void* wq_a, const void* wkv_a, void* out,
                       int M) {
  const int Dq = d->q_lora_rank, NQKV = Dq + d->kv_lora_rank + 64;
  mla::GemmArgs g = gemm_args(x, d->dim, wq_a, d->dim, out, NQKV, adt, M, NQKV, d->dim);
  g.W2 = wkv_a; g.ldw2 = d->dim; g.n_split = Dq;
  return g;
}

// K chunks of the bf16 joint down-projection: its output has few 256x256
// tiles, so it runs split-K into fp32 partials that the two norms sum.
int prefill_qkv_splits(const mla_dims* d, int wdt, int adt, int M) {
  if (wdt != MLA_BF16 || adt != MLA_BF16) return 1;
  const void* aligned = (const void*)(uintptr_t)256;
  return mla::gemm_bf16_splits(qkv_args(d, adt, aligned, aligned, aligned, nullptr, M));
}

// e4m3 joint down-projection on the 256 x 256 e4m3 GEMM: its N = Dq + L + 64
// columns make one tile column of 64 (the k_pe columns) per row of tiles, and
// at M = 16384 those 64 narrow tiles are a whole third round on 8 of each XCD's
// 32 CUs. Computing the k_pe columns as a separate product with its K cut into
// KPE_SPLITS chunks (fp32 partials that the norm pass sums in chunk order) turns
// that round into one of quarter-length tiles on every CU. Used where it
// shortens the launch schedule (whole rounds of 256 workgroups).
// The bf16 joint down-projection (when it is not split-K as a whole) does the
// same when the bf16 GEMM's schedule gains by it (its chunk count is then the
// split-K plan of the 64-column product).
constexpr int KPE_SPLITS = 4, PREFILL_CUS = 256;
int prefill_kpe_splits(const mla_dims* d, int wdt, int adt, int M) {
  if (adt != MLA_BF16 || M < 256) return 0;
  if (wdt == MLA_BF16) {
    if (prefill_qkv_splits(d, wdt, adt, M) > 1) return 0;
    const void* al = (const void*)(uintptr_t)256;
    const mla::GemmArgs full = qkv_args(d, adt, al, al, al, (void*)(uintptr_t)256, M);
    mla::GemmArgs main = full;
    main.N = d->q_lora_rank + d->kv_lora_rank;
    const mla::GemmArgs tail = gemm_args(al, d->dim, al, d->dim, nullptr, 64, adt, M, 64, d->dim);
    const int splits = mla::gemm_bf16_splits(tail);
    if (splits < 2 || splits > 8) return 0;
    const double c_full = mla::gemm_bf16_cost(full, false);
    const double c_split = mla::gemm_bf16_cost(main, false) + mla::gemm_bf16_cost(tail, true);
    return c_split < c_full - 0.25 ? splits : 0;
  }
  if (wdt != MLA_E4M3) return 0;
  const int tm = (M + 255) / 256, tq = (d->q_lora_rank + 255) / 256;
  const int full = tm * (tq + (d->kv_lora_rank + 64 + 255) / 256), main = tm * (tq + (d->kv_lora_rank + 255) / 256);
  const double rounds_full = (full + PREFILL_CUS - 1) / PREFILL_CUS;
  const double rounds_split = (main + PREFILL_CUS - 1) / PREFILL_CUS +
                              (double)((tm * KPE_SPLITS + PREFILL_CUS - 1) / PREFILL_CUS) / KPE_SPLITS;
  return rounds_split < rounds_full - 0.25 ? KPE_SPLITS : 0;
}

// Tk = keys per sequence (T, or start_pos + T with a cache)
size_t prefill_layout(const mla_dims* d, int wdt, int adt, int B, int T, int Tk, int topk, bool own_kvc, void* ws,
                      PrefillWs* out) {
  const size_t M = (size_t)B * T, H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank;
  const size_t es = adt == MLA_F32 ? 4 : 2;
  Carver c(ws);
  PrefillWs p{};
  p.cqkv = wdt == MLA_E4M3 ? nullptr : c.take(M * (Dq + L + 64) * es);   // e4m3: fp32 product in part
  p.cqn = c.take(M * Dq * es);
  p.kvc = own_kvc ? c.take(M * (L + 64) * es) : nullptr;
  const size_t Mp = (size_t)B * pad64(Tk);
  p.q = c.take(M * H * 192 * es);
  p.kn = c.take(Mp * H * 128 * es);
  p.vt = c.take(Mp * H * 128 * es);
  p.kpe = c.take(Mp * 64 * es);
  p.attn = c.take(M * H * 128 * es);
  p.mask = topk > 0 ? c.take((size_t)B * T * ((Tk + 31) / 32) * 4) : nullptr;
  p.qkv_splits = prefill_qkv_splits(d, wdt, adt, (int)M);
  // fp32 input of the norms: split-K partials (bf16), the whole product (e4m3)
  const size_t nparts = wdt == MLA_E4M3 ? 1 : p.qkv_splits > 1 ? p.qkv_splits : 0;
  p.part = nparts ? (float*)c.take(nparts * M * (Dq + L + 64) * 4) : nullptr;
  p.kpe_splits = prefill_kpe_splits(d, wdt, adt, (int)M);
  p.kpe_part = p.kpe_splits ? (float*)c.take((size_t)p.kpe_splits * M * 64 * 4) : nullptr;
  if (wdt == MLA_E4M3) {
    size_t kmax = d->dim;
    if (Dq > kmax) kmax = Dq;
    if (L > kmax) kmax = L;
    if (H * 128 > kmax) kmax = H * 128;
    if (Dq + L > kmax) kmax = Dq + L;   // the norm pass's codes of c_q and the latent side by side
    const size_t rows = M > (size_t)Tk ? M : (size_t)Tk;   // kv_b over a cache runs per sequence
    p.aq = c.take(rows * kmax);
    p.as = c.take(rows * (kmax / 128) * 4);
  }
  if (out) *out = p;
  return c.off;
}

struct DecodeWs {
  void *part, *cqn, *q, *qlat, *o;
  void *attn;          // splits == 1: o_lat [B, H, 512] bf16; else the split partials [splits][B*H][512]
  float* lse;          // splits > 1: [splits][B*H]
  int32_t *keys, *nkeys;   // selected keys: compacted lists [B][DECODE_TOPK_MAX], counts [B]
  int splits;
  void *aq, *as;   // e4m3 weights: the quantised activation of the current projection (x, then c_q)
  void *oq, *os;   // e4m3 weights: o quantised by the un-absorb kernel for wo
};

// Decode projections (M = batch rows): column tile widths and split-K. One
// workgroup per CU fills the chip, and a launch of more than 256 makes a
// second, mostly idle round, so a long-K product takes the largest number of
// K chunks (at most 8) that keeps tiles x chunks <= 256. Measured in the
// DeepSeek-V3.2-Exp decode step at B = 128 (same box, alternating runs):
// q_a|kv_a in 33 x 7 workgroups and q_b in 256 tiles of 96 columns took the
// step from 224 to 216 us (from 33 x 8 and 192 tiles of 128); wo in 32 x 8
// tiles of 224 columns was slower in the step (223 us) than 56 x 4 of 128
// although faster alone.
constexpr int DEC_CUS = 256, DEC_MAX_CHUNKS = 8;
constexpr int DEC_NT_QKV = 64, DEC_NT_QB = 96, DEC_NT_WO = 128, DEC_NT_FP8 = 128;
int dec_chunks(int N, int nt) {
  const int tiles = (N + nt - 1) / nt;
  const int c = DEC_CUS / tiles;
  return c < 1 ? 1 : c > DEC_MAX_CHUNKS ? DEC_MAX_CHUNKS : c;
}
int skinny_splits(int K, int splits);
int skinny_fp8_splits(int K, int splits);

// Column tile width and K chunks of a decode-shaped product with N outputs: a
// narrow output (the joint q_a|kv_a down-projection) takes 64-wide tiles and
// K chunks; a wide one whose tiles alone fill the chip (q_b) one chunk of
// 96-wide (bf16) or 128-wide (e4m3) tiles; the rest (wo) 128-wide tiles and K
// chunks. At the DeepSeek-V3.2-Exp shapes these are the decode step's choices.
struct DecTiling { int nt, chunks; };
DecTiling dec_tiling(int N, bool fp8) {
  if (N <= 4096) return {DEC_NT_QKV, dec_chunks(N, DEC_NT_QKV)};
  const int wide = fp8 ? DEC_NT_FP8 : DEC_NT_QB;
  if ((N + wide - 1) / wide >= (fp8 ? 150 : 200)) return {wide, 1};
  return {DEC_NT_WO, dec_chunks(N, DEC_NT_WO)};
}

// K chunks the q_a|kv_a and wo products of a decode step use (the same
// functions pick them at launch, so the partial buffer always fits)
int dec_qkv_splits(const mla_dims* d, int wdt) {
  const int nqkv = d->q_lora_rank + d->kv_lora_rank + 64;
  return wdt == MLA_E4M3 ? skinny_fp8_splits(d->dim, dec_chunks(nqkv, DEC_NT_QKV))
                         : skinny_splits(d->dim, dec_chunks(nqkv, DEC_NT_QKV));
}
int dec_wo_splits(const mla_dims* d, int wdt) {
  const int K = d->n_heads * 128;
  return wdt == MLA_E4M3 ? skinny_fp8_splits(K, dec_chunks(d->dim, DEC_NT_FP8))
                         : skinny_splits(K, dec_chunks(d->dim, DEC_NT_WO));
}

size_t decode_layout(const mla_dims* d, int wdt, int B, int max_len, void* ws, DecodeWs* out) {
  const size_t H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank;
  Carver c(ws);
  DecodeWs p{};
  const int nqkv = (int)(Dq + L + 64);
  const size_t part_qkv = (size_t)dec_qkv_splits(d, wdt) * B * nqkv,
               part_wo = (size_t)dec_wo_splits(d, wdt) * B * d->dim;
  p.part = c.take((part_qkv > part_wo ? part_qkv : part_wo) * 4);
  p.cqn = c.take((size_t)B * Dq * 2);
  p.q = c.take((size_t)B * H * 192 * 2);
  p.qlat = c.take((size_t)B * H * 576 * 2);
  p.splits = mla::decode_splits(B, (int)H, max_len);
  p.attn = c.take((size_t)p.splits * B * H * 512 * 2);
  p.lse = p.splits > 1 ? (float*)c.take((size_t)p.splits * B * H * 4) : nullptr;
  p.keys = (int32_t*)c.take((size_t)B * mla::DECODE_TOPK_MAX * 4);
  p.nkeys = (int32_t*)c.take((size_t)B * 4);
  if (wdt == MLA_E4M3) {   // widest quantised projection input: x [B, dim] or c_q [B, q_lora_rank]
    const size_t kmax = (size_t)d->dim > Dq ? (size_t)d->dim : Dq;
    p.aq = c.take((size_t)B * kmax);
    p.as = c.take((size_t)B * (kmax / 128) * 4);
    p.oq = c.take((size_t)B * H * 128);
    p.os = c.take((size_t)B * H * 4);
  } else {
    p.o = c.take((size_t)B * H * 128 * 2);
  }
  if (out) *out = p;
  return c.off;
}

struct AbsorbedWs {
  void *cqkv, *cqn, *kvc, *q, *qlat, *olat, *o, *wukt;
  float* part;
  int32_t *keys, *nkeys;   // compacted selections [M][topk], counts [M]
  int qkv_splits;
  float* kpe_part;   // split-K partials of the k_pe columns (prefill_kpe_splits), or NULL
  int kpe_splits;
};

size_t absorbed_layout(const mla_dims* d, int B, int T, int topk, bool own_kvc, void* ws, AbsorbedWs* out) {
  const size_t M = (size_t)B * T, H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank;
  Carver c(ws);
  AbsorbedWs p{};
  p.cqkv = c.take(M * (Dq + L + 64) * 2);
  p.cqn = c.take(M * Dq * 2);
  p.kvc = own_kvc ? c.take(M * (L + 64) * 2) : nullptr;
  p.q = c.take(M * H * 192 * 2);
  p.qlat = c.take(M * H * (L + 64) * 2);
  p.olat = c.take(M * H * L * 2);
  p.o = c.take(M * H * 128 * 2);
  p.wukt = c.take(H * L * 128 * 2);
  p.qkv_splits = prefill_qkv_splits(d, MLA_BF16, MLA_BF16, (int)M);
  p.part = p.qkv_splits > 1 ? (float*)c.take((size_t)p.qkv_splits * M * (Dq + L + 64) * 4) : nullptr;
  p.kpe_splits = prefill_kpe_splits(d, MLA_BF16, MLA_BF16, (int)M);
  p.kpe_part = p.kpe_splits ? (float*)c.take((size_t)p.kpe_splits * M * 64 * 4) : nullptr;
  p.keys = (int32_t*)c.take(M * (size_t)topk * 4);
  p.nkeys = (int32_t*)c.take(M * 4);
  if (out) *out = p;
  return c.off;
}

mla::GemmArgs gemm_args(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int cdt, int M,
                        int N, int K) {
  mla::GemmArgs g{};
  g.A = A; g.lda = lda; g.W = W; g.ldw = ldw; g.W2 = nullptr; g.ldw2 = 0; g.n_split = N;
  g.C = C; g.ldc = ldc; g.c_dtype = cdt; g.M = M; g.N = N; g.K = K; g.batch = 1; g.w_kn = false;
  return g;
}

mla::NormRopeArgs norm_args(const void* in, int64_t ld_in, void* out, int64_t ld_out, int dt, int rows) {
  mla::NormRopeArgs a{};
  a.in = in; a.ld_in = ld_in; a.in_dtype = dt; a.out = out; a.ld_out = ld_out; a.out_dtype = dt; a.rows = rows;
  a.pos_period = 1;
  return a;
}

// operand shapes and alignments the fused q / kv norm kernel takes
bool qkv_norm_ok(const mla::QkvNormArgs& a) {
  const uintptr_t al = (uintptr_t)a.in | (uintptr_t)a.gq | (uintptr_t)a.gkv;
  const uintptr_t al8 = (uintptr_t)a.q_out | (uintptr_t)a.kv_out;
  return (al & 15) == 0 && (al8 & 7) == 0 && a.Dq % 4 == 0 && a.L % 4 == 0 && a.ld_in % 4 == 0 &&
         (a.Dq + a.L + 64) / 4 <= 1024 && a.in_splits <= 64 && (a.split_stride % 4) == 0;
}

// y[M, N] = act[M, K] . W^T for the path's weight format; fp8 quantises act first.
// With kv != nullptr the output goes through the k_nope / v^T split epilogue.
int project(int wdt, int adt, const void* act, int64_t lda, const void* W, const float* Ws,
            const void* W2, const float* W2s, int n_split, void* out, int64_t ldo, int M, int N, int K,
            const PrefillWs* ws, hipStream_t s, const mla::KvSplit* kv = nullptr, const mla::RopeEpi* rope = nullptr,
            bool* roped = nullptr, int cdt = -1, const uint8_t* act_codes = nullptr,
            const float* act_scales = nullptr) {
  const int epi = kv ? mla::EPI_KV_SPLIT : mla::EPI_ROWMAJOR;
  if (roped) *roped = false;
  if (wdt == MLA_E4M3) {
    // the activation's e4m3 codes: made by an earlier pass (act_codes), or quantised here
    if (!act_codes)
      LAUNCH(mla::launch_quant_1x128(act, lda, adt, M, K, (uint8_t*)ws->aq, (float*)ws->as, s), "quant_e4m3_1x128");
    mla::GemmFp8Args g{};
    g.A = act_codes ? act_codes : (const uint8_t*)ws->aq;
    g.a_scale = act_codes ? act_scales : (const float*)ws->as;
    g.W = (const uint8_t*)W; g.w_scale = Ws; g.W2 = (const uint8_t*)W2; g.w2_scale = W2s; g.n_split = n_split;
    g.C = out; g.ldc = ldo; g.c_dtype = cdt < 0 ? adt : cdt; g.M = M; g.N = N; g.K = K;
    g.epi = epi;
    if (kv) g.kv = *kv;
    if (rope) {   // RoPE of the query's rotary slices in the GEMM's epilogue, where it applies
      g.epi = mla::EPI_QROPE; g.rope = *rope;
      if (mla::gemm_fp8_qrope_ok(g) && roped) *roped = true;
      else { g.epi = epi; g.rope = mla::RopeEpi{}; }
    }
    LAUNCH(mla::launch_gemm_fp8(g, s), "gemm_fp8_blockscaled");
    return MLA_OK;
  }
  mla::GemmArgs g = gemm_args(act, lda, W, K, out, ldo, adt, M, N, K);
  g.W2 = W2; g.ldw2 = K; g.n_split = n_split;
  g.epi = epi;
  if (kv) g.kv = *kv;
  if (adt == MLA_F32) LAUNCH(mla::launch_gemm_f32(g, s), "gemm_f32");
  else LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16");
  return MLA_OK;
}

// Decode-shaped product C[z] = A[z] . W[z]^T over rows in chunks of 128; with
// splits > 1 the fp32 partials land in P[split][M][N] (rows at P + m*N).
// K chunk (elements) of a split-K skinny product and the number of chunks it makes.
int skinny_kc(int K, int splits) {
  const int ksteps = K / 64;
  if (splits > ksteps) splits = ksteps;
  return ((ksteps + splits - 1) / splits) * 64;
}
int skinny_splits(int K, int splits) { return (K + skinny_kc(K, splits) - 1) / skinny_kc(K, splits); }

int skinny(const void* A, int64_t lda, int64_t batch_a, const void* W, int64_t ldw, int64_t batch_w,
           const void* W2, int64_t ldw2, int n_split, void* C, int64_t ldc, int64_t batch_c, float* P, int M, int N,
           int K, int batch, int nt, int splits, hipStream_t s) {
  if (K % 64 || K == 0 || lda % 8 || batch_a % 8 || ldw % 8 || batch_w % 8 || (W2 && ldw2 % 8) ||
      ((uintptr_t)A | (uintptr_t)W | (uintptr_t)W2) % 16)
    return fail(MLA_UNSUPPORTED, "decode projection needs K % 64 == 0 and 16-byte aligned rows");
  const int kc = skinny_kc(K, splits);
  splits = skinny_splits(K, splits);
  for (int m0 = 0; m0 < M; m0 += 128) {
    mla::SkinnyArgs g{};
    g.A = (const uint16_t*)A + (int64_t)m0 * lda; g.lda = lda; g.batch_a = batch_a;
    g.W = W; g.ldw = ldw; g.batch_w = batch_w; g.W2 = W2; g.ldw2 = ldw2; g.n_split = n_split;
    g.C = C ? (void*)((uint16_t*)C + (int64_t)m0 * ldc) : nullptr; g.ldc = ldc; g.batch_c = batch_c;
    g.P = P ? P + (int64_t)m0 * N : nullptr; g.ps = (int64_t)M * N;
    g.M = M - m0 < 128 ? M - m0 : 128; g.N = N; g.K = K; g.kc = kc; g.batch = batch;
    LAUNCH(mla::launch_gemm_skinny(g, nt, splits, s), "gemm_skinny");
  }
  return MLA_OK;
}

// e4m3 x e4m3 decode-shaped product: A codes [M, K] (row stride lda bytes) with
// 1x128 scales (row stride lds), W codes with 128x128 block scales (row stride
// ldws = K/128); rows in chunks of 128, split-K chunks of at most 4096.
int skinny_fp8(const void* A, int64_t lda, int64_t batch_a, const float* as, int64_t lds, int64_t batch_as,
               const void* W, int64_t ldw, int64_t batch_w, const float* ws, int ldws, int64_t batch_ws,
               const void* W2, int64_t ldw2, const float* ws2, int n_split, void* C, int64_t ldc, int64_t batch_c,
               float* P, int M, int N, int K, int batch, int nt, int splits, hipStream_t s, uint8_t* qc = nullptr,
               float* qs = nullptr) {
  const int kblocks = K / 128;
  if (splits < (kblocks + 31) / 32) splits = (kblocks + 31) / 32;
  if (splits > kblocks) splits = kblocks;
  const int kc = ((kblocks + splits - 1) / splits) * 128;
  splits = (K + kc - 1) / kc;
  if (splits > 1 && !P) return fail(MLA_INVALID_ARG, "split-K product without a partial buffer");
  for (int m0 = 0; m0 < M; m0 += 128) {
    mla::SkinnyArgs g{};
    g.A = (const uint8_t*)A + (int64_t)m0 * lda; g.lda = lda; g.batch_a = batch_a;
    g.as = as + (int64_t)m0 * lds; g.lds = lds; g.batch_as = batch_as;
    g.W = W; g.ldw = ldw; g.batch_w = batch_w; g.ws = ws; g.ldws = ldws; g.batch_ws = batch_ws;
    g.W2 = W2; g.ldw2 = ldw2; g.ws2 = ws2; g.n_split = W2 ? n_split : N;
    g.C = C ? (void*)((uint16_t*)C + (int64_t)m0 * ldc) : nullptr; g.ldc = ldc; g.batch_c = batch_c;
    g.P = P ? P + (int64_t)m0 * N : nullptr; g.ps = (int64_t)M * N;
    g.M = M - m0 < 128 ? M - m0 : 128; g.N = N; g.K = K; g.kc = kc; g.batch = batch;
    g.qc = qc ? qc + (int64_t)m0 * ldc : nullptr; g.qs = qs ? qs + (int64_t)m0 * (ldc / 128) : nullptr;
    LAUNCH(mla::launch_gemm_skinny_fp8(g, nt, splits, s), "gemm_skinny_fp8");
  }
  return MLA_OK;
}
int skinny_fp8_splits(int K, int splits) {
  const int kblocks = K / 128;
  if (splits < (kblocks + 31) / 32) splits = (kblocks + 31) / 32;
  if (splits > kblocks) splits = kblocks;
  const int kc = ((kblocks + splits - 1) / splits) * 128;
  return (K + kc - 1) / kc;
}

}  // namespace

extern "C" {

const char* mla_version(void) { return "mla-gfx950 0.1.0"; }
const char* mla_last_error(void) { return g_err.c_str(); }

size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t act_dtype, int32_t B, int32_t T,
                                  int32_t topk) {
  if (check_dims(dims) != MLA_OK || B <= 0 || T <= 0) return 0;
  return prefill_layout(dims, weight_dtype, act_dtype, B, T, T, topk, true, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Prefill of T new tokens per sequence at positions P..P+T-1 (P = 0: empty
// cache). cache: [B, cache_bs / (L + 64), L + 64] entries, rows [0, P) given,
// rows [P, P + T) written here; keys are rows 0..P+T-1.
int prefill_impl(const mla_dims* d, const mla_weights* w, const void* x, int32_t adt, int32_t B, int32_t T, int32_t P,
                 void* cache, int64_t cache_bs, bool own_cache, const float* rope_cos, const float* rope_sin,
                 int32_t rope_len, const int32_t* topk_idx, int32_t topk, void* out, void* ws, size_t ws_bytes,
                 void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!w) return fail(MLA_INVALID_ARG, "weights is NULL");
  const int wdt = w->weight_dtype;
  if (!((adt == MLA_F32 && wdt == MLA_F32) || (adt == MLA_BF16 && (wdt == MLA_BF16 || wdt == MLA_E4M3))))
    return fail(MLA_UNSUPPORTED, "supported (act, weight) dtypes: (F32, F32), (BF16, BF16), (BF16, E4M3)");
  if ((rc = check_weights(w, wdt))) return rc;
  if (!x || !out || !rope_cos || !rope_sin) return fail(MLA_INVALID_ARG, "x/out/rope tables must not be NULL");
  if (B <= 0 || T <= 0 || P < 0) return fail(MLA_INVALID_ARG, "B and T must be positive, start_pos >= 0");
  if ((int64_t)B * (P + (int64_t)T) > (1LL << 30)) return fail(MLA_INVALID_ARG, "B*(start_pos+T) too large");
  if (rope_len < P + T) return fail(MLA_INVALID_ARG, "rope_len (%d) < start_pos + T (%d)", rope_len, P + T);
  if ((topk_idx == nullptr) != (topk <= 0)) return fail(MLA_INVALID_ARG, "topk_idx and topk > 0 go together");
  const int H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank, dim = d->dim;
  if (wdt == MLA_E4M3 && (dim % 128 || Dq % 128 || L % 128))
    return fail(MLA_UNSUPPORTED, "e4m3 weights need dim, q_lora_rank, kv_lora_rank multiples of 128");
  const int Tk = P + T;
  PrefillWs p;
  const size_t need = prefill_layout(d, wdt, adt, B, T, Tk, topk, own_cache, ws, &p);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int M = B * T, NQKV = Dq + L + 64;
  void* kvc = own_cache ? p.kvc : cache;
  if (own_cache) cache_bs = (int64_t)T * (L + 64);

  // joint down-projection: [c_q | latent | k_pe] = x . [Wq_a ; Wkv_a]^T, split-K
  // into fp32 partials when its output has too few tiles for the chip
  mla::GemmArgs gq = qkv_args(d, adt, x, w->wq_a, w->wkv_a, p.cqkv, M);
  const bool qkv_split = wdt == MLA_BF16 && p.qkv_splits > 1 && mla::gemm_bf16_splits(gq) == p.qkv_splits;
  // e4m3: the product goes to the norms in fp32 (a bf16 rounding there would
  // move the normalised values that kv_b and q_b quantise again)
  const bool qkv_f32 = qkv_split || wdt == MLA_E4M3;
  const int qkv_nsplit = qkv_split ? p.qkv_splits : 1;
  const size_t es = adt == MLA_F32 ? 4 : 2;
  // the norms read either the projection in the activation type or fp32 (partial) sums
  const void* qkv_in = qkv_f32 ? (const void*)p.part : p.cqkv;
  const size_t qkv_es = qkv_f32 ? 4 : es;
  auto from_qkv = [&](mla::NormRopeArgs& a) {
    if (!qkv_f32) return;
    a.in_dtype = MLA_F32; a.in_splits = qkv_nsplit; a.split_stride = (int64_t)M * NQKV;
  };
  const int Tp = pad64(Tk);
  mla::QkvNormArgs qa{};
  qa.in = qkv_in; qa.ld_in = NQKV; qa.in_dtype = qkv_f32 ? MLA_F32 : adt;
  qa.in_splits = qkv_nsplit; qa.split_stride = (int64_t)M * NQKV;
  qa.rows = M; qa.Dq = Dq; qa.L = L; qa.gq = w->q_norm_w; qa.gkv = w->kv_norm_w; qa.eps = d->rms_eps;
  qa.q_out = p.cqn; qa.ld_q = Dq; qa.kv_out = kvc; qa.ld_kv = L + 64; qa.kv_batch_stride = cache_bs;
  qa.kpe = p.kpe; qa.kpe_tp = Tp;
  qa.cos_tab = rope_cos; qa.sin_tab = rope_sin; qa.rope_len = rope_len; qa.pos_period = T; qa.pos_off = P;
  // e4m3: the norm pass also quantises c_q (q_b's input) and, when kv_b reads
  // exactly these rows, the latent (kv_b's input)
  const bool kv_fresh = P == 0 && cache_bs == (int64_t)T * (L + 64);
  uint8_t* cq_codes = nullptr; float* cq_scales = nullptr;
  uint8_t* kv_codes = nullptr; float* kv_scales = nullptr;
  if (wdt == MLA_E4M3) {
    cq_codes = (uint8_t*)p.aq; cq_scales = (float*)p.as;
    qa.q_codes = cq_codes; qa.q_scales = cq_scales;
    qa.kv_view = true;   // cache entries hold the latent as kv_b's quantiser sees it
    if (kv_fresh) {
      kv_codes = cq_codes + (size_t)M * Dq; kv_scales = cq_scales + (size_t)M * (Dq / 128);
      qa.kv_codes = kv_codes; qa.kv_scales = kv_scales;
    }
  }
  // e4m3 at large M: the k_pe columns as their own split-K product (prefill_kpe_splits)
  const bool kpe_split = p.kpe_part && adt == MLA_BF16 && qkv_norm_ok(qa);
  if (qkv_split) {
    gq.k_splits = p.qkv_splits; gq.part = p.part;
    LAUNCH(mla::launch_gemm_bf16(gq, s), "gemm_bf16(split-K q_a|kv_a)");
  } else if ((rc = project(wdt, adt, x, dim, w->wq_a, w->wq_a_scale, w->wkv_a, w->wkv_a_scale, Dq,
                           qkv_f32 ? (void*)p.part : p.cqkv, NQKV, M, kpe_split ? Dq + L : NQKV, dim, &p, s, nullptr,
                           nullptr, nullptr, qkv_f32 ? MLA_F32 : -1))) {
    return rc;
  }
  if (kpe_split && wdt == MLA_BF16) {   // rows L..L+63 of Wkv_a, split-K into fp32 partials
    mla::GemmArgs g = gemm_args(x, dim, (const uint16_t*)w->wkv_a + (int64_t)L * dim, dim, nullptr, 64, adt, M, 64,
                                dim);
    g.k_splits = p.kpe_splits; g.part = p.kpe_part;
    LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16(k_pe columns, split-K)");
    qa.kpe_in = p.kpe_part; qa.kpe_splits = p.kpe_splits; qa.kpe_split_stride = (int64_t)M * 64;
  } else if (kpe_split) {   // rows L..L+63 of Wkv_a (block row L / 128 of its scales) on x's codes
    mla::GemmFp8Args g{};
    g.A = (const uint8_t*)p.aq; g.a_scale = (const float*)p.as;
    g.W = (const uint8_t*)w->wkv_a + (int64_t)L * dim; g.w_scale = w->wkv_a_scale + (int64_t)(L / 128) * (dim / 128);
    g.C = p.kpe_part; g.ldc = 64; g.c_dtype = MLA_F32; g.M = M; g.N = 64; g.K = dim; g.epi = mla::EPI_ROWMAJOR;
    g.k_splits = p.kpe_splits; g.split_stride = (int64_t)M * 64;
    LAUNCH(mla::launch_gemm_fp8(g, s), "gemm_fp8(k_pe columns, split-K)");
    qa.kpe_in = p.kpe_part; qa.kpe_splits = p.kpe_splits; qa.kpe_split_stride = (int64_t)M * 64;
  }
  if (adt == MLA_BF16 && qkv_norm_ok(qa)) {
    LAUNCH(mla::launch_qkv_norm(qa, s), "qkv_norm");
  } else if (P > 0 || cache_bs != (int64_t)T * (L + 64) || wdt == MLA_E4M3) {
    return fail(MLA_UNSUPPORTED, "prefill over a cache or with e4m3 weights needs bf16 activations and 16-byte "
                                 "aligned norm weights and cache");
  } else {
    cq_codes = nullptr; kv_codes = nullptr;   // the separate norm passes quantise nothing
  {  // q_norm
    mla::NormRopeArgs a = norm_args(qkv_in, NQKV, p.cqn, Dq, adt, M);
    from_qkv(a);
    a.norm_dim = Dq; a.gamma = w->q_norm_w; a.eps = d->rms_eps;
    LAUNCH(mla::launch_rmsnorm_rope(a, s), "rmsnorm_rope(q)");
  }
  {  // kv_norm on the latent, RoPE on the shared key -> [c | k_pe]
    mla::NormRopeArgs a = norm_args((const char*)qkv_in + Dq * qkv_es, NQKV, kvc, L + 64, adt, M);
    from_qkv(a);
    a.norm_dim = L; a.gamma = w->kv_norm_w; a.eps = d->rms_eps;
    a.rope_off = L; a.rope_heads = 1; a.rope_stride = 64;
    a.cos_tab = rope_cos; a.sin_tab = rope_sin; a.rope_len = rope_len; a.pos_period = T;
    a.kpe = p.kpe; a.kpe_tp = Tp;
    LAUNCH(mla::launch_rmsnorm_rope(a, s), "rmsnorm_rope(kv)");
  }
  }
  // q = c_q . Wq_b^T, then RoPE on each head's rotary slice at position P + t
  // (in the GEMM's epilogue on the bf16 and e4m3 paths, a separate pass otherwise)
  const float* cos_p = rope_cos + (int64_t)P * 32;
  const float* sin_p = rope_sin + (int64_t)P * 32;
  mla::GemmArgs gr = gemm_args(p.cqn, Dq, w->wq_b, Dq, p.q, H * 192, adt, M, H * 192, Dq);
  gr.epi = mla::EPI_QROPE; gr.rope = {cos_p, sin_p, T};
  if (wdt == MLA_BF16 && adt == MLA_BF16 && mla::gemm_bf16_qrope_ok(gr)) {
    LAUNCH(mla::launch_gemm_bf16(gr, s), "gemm_bf16(q_b + RoPE)");
  } else {
    bool roped = false;
    if ((rc = project(wdt, adt, p.cqn, Dq, w->wq_b, w->wq_b_scale, nullptr, nullptr, H * 192, p.q, H * 192, M,
                      H * 192, Dq, &p, s, nullptr, &gr.rope, &roped, -1, cq_codes, cq_scales)))
      return rc;
    if (!roped) {
      mla::NormRopeArgs a = norm_args(p.q, H * 192, p.q, H * 192, adt, M);
      a.rope_off = 128; a.rope_heads = H; a.rope_stride = 192;
      a.cos_tab = cos_p; a.sin_tab = sin_p; a.rope_len = rope_len - P; a.pos_period = T;
      LAUNCH(mla::launch_rmsnorm_rope(a, s), "rmsnorm_rope(q_pe)");
    }
  }
  // per head [k_nope | v] = c . Wkv_b^T over all Tk keys, stored as
  // k_nope [B,H,Tp,128] and v^T [B,H,128,Tp]; the cached keys' k_pe joins the new ones
  LAUNCH(mla::launch_zero_kv_padding(p.kn, p.vt, p.kpe, B, H, Tk, Tp, (int)es, s), "zero_kv_padding");
  LAUNCH(mla::launch_gather_kpe(kvc, cache_bs, L + 64, L, B, P, p.kpe, Tp, s), "gather_kpe");
  if (kv_fresh) {   // one launch over the B*T contiguous entries
    const mla::KvSplit split{p.vt, T, Tp, H};
    if ((rc = project(wdt, adt, kvc, L + 64, w->wkv_b, w->wkv_b_scale, nullptr, nullptr, H * 256, p.kn, 0, M,
                      H * 256, L, &p, s, &split, nullptr, nullptr, -1, kv_codes, kv_scales)))
      return rc;
  } else {
    for (int b = 0; b < B; ++b) {   // the sequences' cache rows are cache_bs apart
      const mla::KvSplit split{(char*)p.vt + (size_t)b * H * 128 * Tp * es, Tk, Tp, H};
      if ((rc = project(wdt, adt, (const char*)kvc + (size_t)b * cache_bs * es, L + 64, w->wkv_b, w->wkv_b_scale,
                        nullptr, nullptr, H * 256, (char*)p.kn + (size_t)b * H * Tp * 128 * es, 0, Tk, H * 256, L,
                        &p, s, &split)))
        return rc;
    }
  }
  if (topk > 0)
    LAUNCH(mla::launch_topk_bitmask(topk_idx, B, T, topk, P, Tk, (uint32_t*)p.mask, s), "topk_to_bitmask");
  mla::PrefillAttnArgs at{};
  at.q = p.q; at.kn = p.kn; at.vt = p.vt; at.kpe = p.kpe;
  at.mask = (const uint32_t*)p.mask; at.out = p.attn; at.B = B; at.T = T; at.Tp = Tp; at.H = H; at.P = P;
  at.scale = d->softmax_scale;
  const bool o_codes = wdt == MLA_E4M3 && adt == MLA_BF16;   // wo's e4m3 input straight from the attention
  if (o_codes) { at.oq = (uint8_t*)p.aq; at.os = (float*)p.as; }
  if (adt == MLA_F32) LAUNCH(mla::launch_prefill_attn_f32(at, s), "prefill_attn_f32");
  else LAUNCH(mla::launch_prefill_attn_bf16(at, s), "prefill_attn");
  // out = o . Wo^T
  return project(wdt, adt, p.attn, H * 128, w->wo, w->wo_scale, nullptr, nullptr, dim, out, dim, M, dim, H * 128,
                 &p, s, nullptr, nullptr, nullptr, -1, o_codes ? (const uint8_t*)p.aq : nullptr,
                 o_codes ? (const float*)p.as : nullptr);
}

}  // namespace

extern "C" {

int mla_prefill(const mla_dims* d, const mla_weights* w, const void* x, int32_t adt, int32_t B, int32_t T,
                const float* rope_cos, const float* rope_sin, int32_t rope_len, const int32_t* topk_idx,
                int32_t topk, void* out, void* kv_cache_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  const int L = d ? d->kv_lora_rank : 0;
  return prefill_impl(d, w, x, adt, B, T, 0, kv_cache_out, (int64_t)T * (L + 64), kv_cache_out == nullptr, rope_cos,
                      rope_sin, rope_len, topk_idx, topk, out, ws, ws_bytes, stream);
}

size_t mla_prefill_cached_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t B, int32_t T,
                                         int32_t start_pos, int32_t topk) {
  if (check_dims(dims) != MLA_OK || B <= 0 || T <= 0 || start_pos < 0) return 0;
  return prefill_layout(dims, weight_dtype, MLA_BF16, B, T, start_pos + T, topk, false, nullptr, nullptr);
}

int mla_prefill_cached(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t T,
                       int32_t start_pos, void* kv_cache, int32_t max_len, const float* rope_cos,
                       const float* rope_sin, int32_t rope_len, const int32_t* topk_idx, int32_t topk, void* out,
                       void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!d) return fail(MLA_INVALID_ARG, "dims is NULL");
  if (!kv_cache) return fail(MLA_INVALID_ARG, "kv_cache must not be NULL");
  if (start_pos < 0 || T <= 0 || max_len <= 0 || (int64_t)start_pos + T > max_len)
    return fail(MLA_INVALID_ARG, "need 0 <= start_pos and start_pos + T (%lld) <= max_len (%d)",
                (long long)start_pos + T, max_len);
  if ((uintptr_t)kv_cache & 15) return fail(MLA_UNSUPPORTED, "kv_cache must be 16-byte aligned");
  return prefill_impl(d, w, x, MLA_BF16, B, T, start_pos, kv_cache, (int64_t)max_len * (d->kv_lora_rank + 64), false,
                      rope_cos, rope_sin, rope_len, topk_idx, topk, out, ws, ws_bytes, stream);
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t weight_dtype, int32_t B, int32_t max_len) {
  if (check_dims(dims) != MLA_OK || B <= 0 || max_len <= 0 ||
      (weight_dtype != MLA_BF16 && weight_dtype != MLA_E4M3))
    return 0;
  return decode_layout(dims, weight_dtype, B, max_len, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Decode step; with topk_idx the attention covers only the listed positions.
int decode_impl(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, void* kv_cache, int32_t max_len,
                const int32_t* cache_len, const int32_t* topk_idx, int32_t topk, const float* rope_cos,
                const float* rope_sin, int32_t rope_len, void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!w) return fail(MLA_INVALID_ARG, "weights is NULL");
  const int wdt = w->weight_dtype;
  if (wdt != MLA_BF16 && wdt != MLA_E4M3) return fail(MLA_UNSUPPORTED, "decode needs bf16 or e4m3 weights");
  if ((rc = check_weights(w, wdt))) return rc;
  if (d->kv_lora_rank != 512) return fail(MLA_UNSUPPORTED, "decode needs kv_lora_rank = 512");
  if (d->n_heads % 64) return fail(MLA_UNSUPPORTED, "decode needs n_heads to be a multiple of 64");
  if (!x || !kv_cache || !cache_len || !rope_cos || !rope_sin || !out)
    return fail(MLA_INVALID_ARG, "x/kv_cache/cache_len/rope tables/out must not be NULL");
  if (B <= 0 || max_len <= 0) return fail(MLA_INVALID_ARG, "B and max_len must be positive");
  if (max_len > MAX_CACHE_LEN) return fail(MLA_INVALID_ARG, "max_len (%d) above %d", max_len, MAX_CACHE_LEN);
  if (rope_len < max_len) return fail(MLA_INVALID_ARG, "rope_len (%d) < max_len (%d)", rope_len, max_len);
  if (((uintptr_t)x | (uintptr_t)kv_cache | (uintptr_t)out) & 15)
    return fail(MLA_UNSUPPORTED, "decode needs 16-byte aligned x, kv_cache and out");
  DecodeWs p;
  const size_t need = decode_layout(d, wdt, B, max_len, ws, &p);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank, dim = d->dim, NQKV = Dq + L + 64;

  if (dim % 64 || Dq % 64) return fail(MLA_UNSUPPORTED, "decode needs dim and q_lora_rank multiples of 64");
  const bool fp8 = wdt == MLA_E4M3;
  if (fp8 && (dim % 128 || Dq % 128))
    return fail(MLA_UNSUPPORTED, "e4m3 decode needs dim and q_lora_rank multiples of 128");
  float* part = (float*)p.part;
  uint8_t* aq = (uint8_t*)p.aq;
  float* as = (float*)p.as;
  // [c_q | latent | k_pe] = x . [Wq_a ; Wkv_a]^T as split-K partials, summed by the norms
  const int splits_qkv = dec_qkv_splits(d, wdt);
  if (fp8) {   // x quantised in 1x128 groups first
    LAUNCH(mla::launch_quant_1x128(x, dim, MLA_BF16, B, dim, aq, as, s), "quant_e4m3_1x128(x)");
    if ((rc = skinny_fp8(aq, dim, 0, as, dim / 128, 0, w->wq_a, dim, 0, w->wq_a_scale, dim / 128, 0, w->wkv_a, dim,
                         w->wkv_a_scale, Dq, nullptr, 0, 0, part, B, NQKV, dim, 1, DEC_NT_QKV,
                         dec_chunks(NQKV, DEC_NT_QKV), s)))
      return rc;
  } else if ((rc = skinny(x, dim, 0, w->wq_a, dim, 0, w->wkv_a, dim, Dq, nullptr, 0, 0, part, B, NQKV, dim, 1,
                          DEC_NT_QKV, dec_chunks(NQKV, DEC_NT_QKV), s))) {
    return rc;
  }
  {  // q_norm, kv_norm and RoPE of k_pe; the new [latent | k_pe] lands directly in cache row cache_len[b]
    mla::QkvNormArgs a{};
    a.in = part; a.ld_in = NQKV; a.in_dtype = MLA_F32; a.in_splits = splits_qkv; a.split_stride = (int64_t)B * NQKV;
    a.rows = B; a.Dq = Dq; a.L = L; a.gq = w->q_norm_w; a.gkv = w->kv_norm_w; a.eps = d->rms_eps;
    a.q_out = p.cqn; a.ld_q = Dq;
    a.kv_out = kv_cache; a.ld_kv = (int64_t)max_len * (L + 64); a.kv_pos_stride = L + 64; a.kv_pos_max = max_len;
    a.cos_tab = rope_cos; a.sin_tab = rope_sin; a.rope_len = max_len; a.pos = cache_len;
    if (fp8) {
      a.q_codes = aq; a.q_scales = as;   // q_b's input, quantised in the same pass
      a.kv_view = true;                  // the entry as kv_b's quantiser sees it
    }
    if (!qkv_norm_ok(a)) return fail(MLA_UNSUPPORTED, "decode needs 16-byte aligned norm weights");
    LAUNCH(mla::launch_qkv_norm(a, s), "qkv_norm -> cache");
  }
  // q = c_q . Wq_b^T
  if (fp8) {
    if ((rc = skinny_fp8(aq, Dq, 0, as, Dq / 128, 0, w->wq_b, Dq, 0, w->wq_b_scale, Dq / 128, 0, nullptr, 0, nullptr,
                         H * 192, p.q, H * 192, 0, nullptr, B, H * 192, Dq, 1, 128, 1, s)))
      return rc;
  } else if ((rc = skinny(p.cqn, Dq, 0, w->wq_b, Dq, 0, nullptr, 0, H * 192, p.q, H * 192, 0, nullptr, B, H * 192, Dq,
                          1, DEC_NT_QB, 1, s))) {
    return rc;
  }
  // q_lat[b, h] = [q_nope[b, h] . W_UK_h | RoPE(q_pe[b, h])]  (W_UK_h = Wkv_b rows [256h, 256h+128))
  LAUNCH(mla::launch_decode_absorb(p.q, w->wkv_b, fp8 ? w->wkv_b_scale : nullptr, p.qlat, cache_len, rope_cos,
                                   rope_sin, B, H, max_len, s),
         "decode_absorb");
  if (topk_idx)   // each row's selection as its ascending, duplicate-free list of live positions
    LAUNCH(mla::launch_decode_compact(topk_idx, topk, cache_len, 0, B, max_len, p.keys, mla::DECODE_TOPK_MAX, p.nkeys,
                                      s),
           "decode_compact");
  {
    mla::DecodeAttnArgs a{};
    a.qlat = p.qlat; a.cache = kv_cache; a.cache_len = cache_len;
    a.R = B; a.H = H; a.max_len = max_len; a.scale = d->softmax_scale;
    if (topk_idx) { a.keys = p.keys; a.nkeys = p.nkeys; a.kstride = mla::DECODE_TOPK_MAX; }
    a.splits = p.splits;
    if (p.splits == 1) a.olat = p.attn;
    else { a.part = p.attn; a.lse = p.lse; }
    LAUNCH(mla::launch_decode_attn(a, s), "decode_attn");
  }
  {  // o[b, h] = W_UV_h . o_lat[b, h] (splits merged in order); e4m3: o leaves as wo's quantised input
    mla::UnabsorbArgs u{};
    u.part = p.attn; u.lse = p.lse; u.splits = p.splits;
    u.wkv_b = w->wkv_b; u.w_scale = fp8 ? w->wkv_b_scale : nullptr;
    u.ldo = (int64_t)H * 128;
    if (fp8) { u.oq = (uint8_t*)p.oq; u.os = (float*)p.os; }
    else u.o = p.o;
    u.B = B; u.H = H;
    LAUNCH(mla::launch_decode_unabsorb(u, s), "decode_unabsorb");
  }
  // out = o . Wo^T (split-K, then a fixed-order sum)
  if (fp8) {
    if ((rc = skinny_fp8(p.oq, H * 128, 0, (const float*)p.os, H, 0, w->wo, H * 128, 0, w->wo_scale, H, 0, nullptr, 0,
                         nullptr, dim, nullptr, 0, 0, part, B, dim, H * 128, 1, DEC_NT_FP8,
                         dec_chunks(dim, DEC_NT_FP8), s)))
      return rc;
  } else if ((rc = skinny(p.o, H * 128, 0, w->wo, H * 128, 0, nullptr, 0, dim, nullptr, 0, 0, part, B, dim, H * 128,
                          1, DEC_NT_WO, dec_chunks(dim, DEC_NT_WO), s))) {
    return rc;
  }
  LAUNCH(mla::launch_splitk_reduce(part, dec_wo_splits(d, wdt), B, dim, out, dim, s), "splitk_reduce(wo)");
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, void* kv_cache, int32_t max_len,
               const int32_t* cache_len, const float* rope_cos, const float* rope_sin, int32_t rope_len, void* out,
               void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  return decode_impl(d, w, x, B, kv_cache, max_len, cache_len, nullptr, 0, rope_cos, rope_sin, rope_len, out, ws,
                     ws_bytes, stream);
}

int mla_decode_sparse(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, void* kv_cache,
                      int32_t max_len, const int32_t* cache_len, const int32_t* topk_idx, int32_t topk,
                      const float* rope_cos, const float* rope_sin, int32_t rope_len, void* out, void* ws,
                      size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!topk_idx) return fail(MLA_INVALID_ARG, "topk_idx must not be NULL");
  if (topk <= 0 || topk > mla::DECODE_TOPK_MAX)
    return fail(MLA_UNSUPPORTED, "topk must be in [1, %d]", mla::DECODE_TOPK_MAX);
  return decode_impl(d, w, x, B, kv_cache, max_len, cache_len, topk_idx, topk, rope_cos, rope_sin, rope_len, out, ws,
                     ws_bytes, stream);
}

size_t mla_prefill_absorbed_workspace_size(const mla_dims* dims, int32_t B, int32_t T, int32_t topk) {
  if (check_dims(dims) != MLA_OK || B <= 0 || T <= 0 || topk <= 0 || topk > mla::DECODE_TOPK_MAX) return 0;
  return absorbed_layout(dims, B, T, topk, true, nullptr, nullptr);
}

int mla_prefill_absorbed(const mla_dims* d, const mla_weights* w, const void* x, int32_t B, int32_t T,
                         const float* rope_cos, const float* rope_sin, int32_t rope_len, const int32_t* topk_idx,
                         int32_t topk, void* out, void* kv_cache_out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_dims(d);
  if (rc) return rc;
  if ((rc = check_weights(w, MLA_BF16))) return rc;
  if (d->kv_lora_rank != 512) return fail(MLA_UNSUPPORTED, "the absorbed prefill needs kv_lora_rank = 512");
  if (d->n_heads % 64) return fail(MLA_UNSUPPORTED, "the absorbed prefill needs n_heads a multiple of 64");
  if (!x || !out || !rope_cos || !rope_sin || !topk_idx)
    return fail(MLA_INVALID_ARG, "x/out/rope tables/topk_idx must not be NULL");
  if (B <= 0 || T <= 0) return fail(MLA_INVALID_ARG, "B and T must be positive");
  if ((int64_t)B * T > (1LL << 24)) return fail(MLA_INVALID_ARG, "B*T too large");
  if (rope_len < T) return fail(MLA_INVALID_ARG, "rope_len (%d) < T (%d)", rope_len, T);
  if (topk <= 0 || topk > mla::DECODE_TOPK_MAX)
    return fail(MLA_UNSUPPORTED, "topk must be in [1, %d]", mla::DECODE_TOPK_MAX);
  AbsorbedWs p;
  if (T > MAX_CACHE_LEN) return fail(MLA_INVALID_ARG, "T (%d) above %d", T, MAX_CACHE_LEN);
  if (((uintptr_t)x | (uintptr_t)out | (uintptr_t)kv_cache_out) & 15)
    return fail(MLA_UNSUPPORTED, "the absorbed prefill needs 16-byte aligned x, out and kv_cache_out");
  const size_t need = absorbed_layout(d, B, T, topk, kv_cache_out == nullptr, ws, &p);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int H = d->n_heads, Dq = d->q_lora_rank, L = d->kv_lora_rank, dim = d->dim, NQKV = Dq + L + 64, M = B * T;
  void* kvc = kv_cache_out ? kv_cache_out : p.kvc;
  const uint16_t* wkv_b = (const uint16_t*)w->wkv_b;

  // [c_q | latent | k_pe] and the norms exactly as in prefill: the cache entries and c_q
  mla::GemmArgs gq = qkv_args(d, MLA_BF16, x, w->wq_a, w->wkv_a, p.cqkv, M);
  const bool qkv_split = p.qkv_splits > 1 && mla::gemm_bf16_splits(gq) == p.qkv_splits;
  const bool kpe_split = !qkv_split && p.kpe_part;
  if (qkv_split) {
    gq.k_splits = p.qkv_splits; gq.part = p.part;
    LAUNCH(mla::launch_gemm_bf16(gq, s), "gemm_bf16(split-K q_a|kv_a)");
  } else {
    if (kpe_split) gq.N = Dq + L;   // the k_pe columns follow as their own split-K product
    LAUNCH(mla::launch_gemm_bf16(gq, s), "gemm_bf16(q_a|kv_a)");
  }
  if (kpe_split) {
    mla::GemmArgs g = gemm_args(x, d->dim, (const uint16_t*)w->wkv_a + (int64_t)L * d->dim, d->dim, nullptr, 64,
                                MLA_BF16, M, 64, d->dim);
    g.k_splits = p.kpe_splits; g.part = p.kpe_part;
    LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16(k_pe columns, split-K)");
  }
  mla::QkvNormArgs qa{};
  if (kpe_split) { qa.kpe_in = p.kpe_part; qa.kpe_splits = p.kpe_splits; qa.kpe_split_stride = (int64_t)M * 64; }
  qa.in = qkv_split ? (const void*)p.part : p.cqkv; qa.ld_in = NQKV; qa.in_dtype = qkv_split ? MLA_F32 : MLA_BF16;
  qa.in_splits = qkv_split ? p.qkv_splits : 1; qa.split_stride = (int64_t)M * NQKV;
  qa.rows = M; qa.Dq = Dq; qa.L = L; qa.gq = w->q_norm_w; qa.gkv = w->kv_norm_w; qa.eps = d->rms_eps;
  qa.q_out = p.cqn; qa.ld_q = Dq; qa.kv_out = kvc; qa.ld_kv = L + 64;
  qa.cos_tab = rope_cos; qa.sin_tab = rope_sin; qa.rope_len = rope_len; qa.pos_period = T;
  if (!qkv_norm_ok(qa)) return fail(MLA_UNSUPPORTED, "the absorbed prefill needs 16-byte aligned norm weights");
  LAUNCH(mla::launch_qkv_norm(qa, s), "qkv_norm");
  // q = c_q . Wq_b^T with the rotary slices rotated at position t
  mla::GemmArgs gr = gemm_args(p.cqn, Dq, w->wq_b, Dq, p.q, H * 192, MLA_BF16, M, H * 192, Dq);
  gr.epi = mla::EPI_QROPE; gr.rope = {rope_cos, rope_sin, T};
  if (mla::gemm_bf16_qrope_ok(gr)) {
    LAUNCH(mla::launch_gemm_bf16(gr, s), "gemm_bf16(q_b + RoPE)");
  } else {
    gr.epi = mla::EPI_ROWMAJOR;
    LAUNCH(mla::launch_gemm_bf16(gr, s), "gemm_bf16(q_b)");
    mla::NormRopeArgs a = norm_args(p.q, H * 192, p.q, H * 192, MLA_BF16, M);
    a.rope_off = 128; a.rope_heads = H; a.rope_stride = 192;
    a.cos_tab = rope_cos; a.sin_tab = rope_sin; a.rope_len = rope_len; a.pos_period = T;
    LAUNCH(mla::launch_rmsnorm_rope(a, s), "rmsnorm_rope(q_pe)");
  }
  // q_lat[m, h] = [q_nope[m, h] . W_UK_h | q_pe[m, h]]: per head, W_UK_h = Wkv_b rows
  // [256h, 256h+128) transposed once per call to the [N = 512, K = 128] operand
  // of the big-tile GEMM
  {
    LAUNCH(mla::launch_transpose16(wkv_b, L, 256 * (int64_t)L, (uint16_t*)p.wukt, 128, (int64_t)L * 128, 128, L, H, s),
           "transpose W_UK");
    mla::GemmArgs g = gemm_args(p.q, H * 192, p.wukt, 128, p.qlat, H * 576, MLA_BF16, M, L, 128);
    g.batch = H; g.batch_a = 192; g.batch_w = (int64_t)L * 128; g.batch_c = 576;
    LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16(absorb W_UK)");
    LAUNCH(mla::launch_copy_rows((const uint16_t*)p.q + 128, 192, (uint16_t*)p.qlat + L, 576, (int64_t)M * H, 64, s),
           "copy q_pe");
  }
  // attention of every token over its selected cache entries (compacted to an
  // ascending, duplicate-free list first), in the latent space; one key run per token
  LAUNCH(mla::launch_decode_compact(topk_idx, topk, nullptr, T, M, T, p.keys, topk, p.nkeys, s), "compact selection");
  {
    mla::DecodeAttnArgs a{};
    a.qlat = p.qlat; a.cache = kvc; a.cache_len = nullptr; a.olat = p.olat; a.splits = 1;
    a.R = M; a.H = H; a.max_len = T; a.scale = d->softmax_scale;
    a.keys = p.keys; a.nkeys = p.nkeys; a.kstride = topk; a.rows_per_seq = T;
    LAUNCH(mla::launch_decode_attn(a, s), "sparse latent attention");
  }
  // o[m, h] = W_UV_h . o_lat[m, h] per head (W_UV_h = Wkv_b rows [256h+128, 256h+256)), then wo
  {
    mla::GemmArgs g = gemm_args(p.olat, H * (int64_t)L, wkv_b + 128 * (int64_t)L, L, p.o, H * 128, MLA_BF16, M, 128,
                                L);
    g.batch = H; g.batch_a = L; g.batch_w = 256 * (int64_t)L; g.batch_c = 128;
    LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16(W_UV)");
  }
  LAUNCH(mla::launch_gemm_bf16(gemm_args(p.o, H * 128, w->wo, H * 128, out, dim, MLA_BF16, M, dim, H * 128), s),
         "gemm_bf16(wo)");
  return MLA_OK;
}

// ---------------------------------------------------------------------------
// building blocks

int gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int32_t c_dtype,
              int32_t M, int32_t N, int32_t K, void* stream) {
  g_err.clear();
  if (!A || !W || !C) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M < 0 || N < 0 || K <= 0) return fail(MLA_INVALID_ARG, "bad sizes M=%d N=%d K=%d", M, N, K);
  if (c_dtype != MLA_F32 && c_dtype != MLA_BF16) return fail(MLA_UNSUPPORTED, "c_dtype must be F32 or BF16");
  if (K % 8 || lda % 8 || ldw % 8 || lda < K || ldw < K || ldc < N)
    return fail(MLA_UNSUPPORTED, "need K, lda, ldw multiples of 8, lda/ldw >= K, ldc >= N");
  if (((uintptr_t)A | (uintptr_t)W) & 15) return fail(MLA_UNSUPPORTED, "A and W must be 16-byte aligned");
  if (M == 0 || N == 0) return MLA_OK;
  mla::GemmArgs g = gemm_args(A, lda, W, ldw, C, ldc, c_dtype, M, N, K);
  LAUNCH(mla::launch_gemm_bf16(g, (hipStream_t)stream), "gemm_bf16");
  return MLA_OK;
}

int gemm_f32(const float* A, int64_t lda, const float* W, int64_t ldw, float* C, int64_t ldc, int32_t M, int32_t N,
             int32_t K, void* stream) {
  g_err.clear();
  if (!A || !W || !C) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M < 0 || N < 0 || K <= 0 || lda < K || ldw < K || ldc < N) return fail(MLA_INVALID_ARG, "bad sizes");
  if (M == 0 || N == 0) return MLA_OK;
  mla::GemmArgs g = gemm_args(A, lda, W, ldw, C, ldc, MLA_F32, M, N, K);
  LAUNCH(mla::launch_gemm_f32(g, (hipStream_t)stream), "gemm_f32");
  return MLA_OK;
}

int gemm_fp8_blockscaled(const uint8_t* Aq, const float* a_scale, const uint8_t* Wq, const float* w_scale, void* C,
                         int64_t ldc, int32_t c_dtype, int32_t M, int32_t N, int32_t K, void* stream) {
  g_err.clear();
  if (!Aq || !a_scale || !Wq || !w_scale || !C) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M < 0 || N < 0 || K <= 0 || ldc < N) return fail(MLA_INVALID_ARG, "bad sizes");
  if (K % 128) return fail(MLA_UNSUPPORTED, "K must be a multiple of 128");
  if (c_dtype != MLA_F32 && c_dtype != MLA_BF16) return fail(MLA_UNSUPPORTED, "c_dtype must be F32 or BF16");
  if (((uintptr_t)Aq | (uintptr_t)Wq) & 15) return fail(MLA_UNSUPPORTED, "Aq and Wq must be 16-byte aligned");
  if (M == 0 || N == 0) return MLA_OK;
  mla::GemmFp8Args g{};
  g.A = Aq; g.a_scale = a_scale; g.W = Wq; g.w_scale = w_scale; g.W2 = nullptr; g.w2_scale = nullptr; g.n_split = N;
  g.C = C; g.ldc = ldc; g.c_dtype = c_dtype; g.M = M; g.N = N; g.K = K;
  LAUNCH(mla::launch_gemm_fp8(g, (hipStream_t)stream), "gemm_fp8_blockscaled");
  return MLA_OK;
}

size_t gemm_decode_workspace_size(int32_t weight_dtype, int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || (weight_dtype != MLA_BF16 && weight_dtype != MLA_E4M3)) return 0;
  const bool fp8 = weight_dtype == MLA_E4M3;
  if (K % (fp8 ? 128 : 64)) return 0;
  const DecTiling t = dec_tiling(N, fp8);
  const int splits = fp8 ? skinny_fp8_splits(K, t.chunks) : skinny_splits(K, t.chunks);
  return splits > 1 ? align256((size_t)splits * (M < 128 ? M : 128) * N * 4) : 256;
}

int gemm_bf16_decode(const void* A, const void* W, void* C, int32_t M, int32_t N, int32_t K, void* ws,
                     size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!A || !W || !C) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M <= 0 || M > 128 || N <= 0 || K <= 0) return fail(MLA_INVALID_ARG, "need 0 < M <= 128, N > 0, K > 0");
  if (K % 64) return fail(MLA_UNSUPPORTED, "K must be a multiple of 64");
  if (((uintptr_t)A | (uintptr_t)W | (uintptr_t)C) & 15) return fail(MLA_UNSUPPORTED, "A, W, C must be 16-byte aligned");
  const size_t need = gemm_decode_workspace_size(MLA_BF16, M, N, K);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const DecTiling t = dec_tiling(N, false);
  const int splits = skinny_splits(K, t.chunks);
  int rc = skinny(A, K, 0, W, K, 0, nullptr, 0, N, splits > 1 ? nullptr : C, N, 0, splits > 1 ? (float*)ws : nullptr,
                  M, N, K, 1, t.nt, t.chunks, s);
  if (rc) return rc;
  if (splits > 1) LAUNCH(mla::launch_splitk_reduce((const float*)ws, splits, M, N, C, N, s), "splitk_reduce");
  return MLA_OK;
}

int gemm_fp8_decode(const uint8_t* Aq, const float* a_scale, const uint8_t* Wq, const float* w_scale, void* C,
                    int32_t M, int32_t N, int32_t K, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!Aq || !a_scale || !Wq || !w_scale || !C) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M <= 0 || M > 128 || N <= 0 || K <= 0) return fail(MLA_INVALID_ARG, "need 0 < M <= 128, N > 0, K > 0");
  if (K % 128) return fail(MLA_UNSUPPORTED, "K must be a multiple of 128");
  if (((uintptr_t)Aq | (uintptr_t)Wq | (uintptr_t)C) & 15)
    return fail(MLA_UNSUPPORTED, "Aq, Wq, C must be 16-byte aligned");
  const size_t need = gemm_decode_workspace_size(MLA_E4M3, M, N, K);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const DecTiling t = dec_tiling(N, true);
  const int splits = skinny_fp8_splits(K, t.chunks);
  int rc = skinny_fp8(Aq, K, 0, a_scale, K / 128, 0, Wq, K, 0, w_scale, K / 128, 0, nullptr, 0, nullptr, N,
                      splits > 1 ? nullptr : C, N, 0, splits > 1 ? (float*)ws : nullptr, M, N, K, 1, t.nt, t.chunks, s);
  if (rc) return rc;
  if (splits > 1) LAUNCH(mla::launch_splitk_reduce((const float*)ws, splits, M, N, C, N, s), "splitk_reduce");
  return MLA_OK;
}

int rmsnorm_rope(const void* in, int64_t ld_in, int32_t in_dtype, int32_t rows, int32_t norm_dim, const float* gamma,
                 float eps, int32_t rope_off, int32_t rope_heads, int32_t rope_stride, const float* cos_tab,
                 const float* sin_tab, int32_t rope_len, const int32_t* pos, int32_t pos_period, void* out,
                 int64_t ld_out, int32_t out_dtype, void* stream) {
  g_err.clear();
  if (!in || !out) return fail(MLA_INVALID_ARG, "NULL in/out");
  if ((in_dtype != MLA_F32 && in_dtype != MLA_BF16) || (out_dtype != MLA_F32 && out_dtype != MLA_BF16))
    return fail(MLA_UNSUPPORTED, "dtypes must be F32 or BF16");
  if (rows < 0 || norm_dim < 0 || rope_heads < 0) return fail(MLA_INVALID_ARG, "negative size");
  if (norm_dim > 0 && !gamma) return fail(MLA_INVALID_ARG, "gamma is NULL");
  if (rope_heads > 0) {
    if (!cos_tab || !sin_tab || rope_len <= 0) return fail(MLA_INVALID_ARG, "rope tables missing");
    if (!pos && (pos_period <= 0 || pos_period > rope_len)) return fail(MLA_INVALID_ARG, "bad pos_period");
    if (rope_off < 0 || (rope_heads > 1 && rope_stride < 64)) return fail(MLA_INVALID_ARG, "bad rope layout");
  }
  int64_t span = norm_dim;
  if (rope_heads > 0) {
    int64_t e = rope_off + (int64_t)(rope_heads - 1) * rope_stride + 64;
    if (e > span) span = e;
  }
  if (ld_in < span || ld_out < span) return fail(MLA_INVALID_ARG, "ld_in/ld_out shorter than the row span");
  mla::NormRopeArgs a{};
  a.in = in; a.ld_in = ld_in; a.in_dtype = in_dtype; a.out = out; a.ld_out = ld_out; a.out_dtype = out_dtype;
  a.rows = rows; a.norm_dim = norm_dim; a.gamma = gamma; a.eps = eps;
  a.rope_off = rope_off; a.rope_heads = rope_heads; a.rope_stride = rope_stride;
  a.cos_tab = cos_tab; a.sin_tab = sin_tab; a.rope_len = rope_len; a.pos = pos; a.pos_period = pos_period > 0 ? pos_period : 1;
  LAUNCH(mla::launch_rmsnorm_rope(a, (hipStream_t)stream), "rmsnorm_rope");
  return MLA_OK;
}

int mla_prefill_attention(const void* q, const void* k_nope, const void* v_t, const void* k_pe, const uint32_t* mask,
                          void* out, int32_t dtype, int32_t B, int32_t T, int32_t H, float scale, void* stream) {
  g_err.clear();
  if (!q || !k_nope || !v_t || !k_pe || !out) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (B <= 0 || T <= 0 || H <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  if (dtype != MLA_BF16 && dtype != MLA_F32) return fail(MLA_UNSUPPORTED, "dtype must be BF16 or F32");
  hipStream_t s = (hipStream_t)stream;
  const int Tp = pad64(T);
  LAUNCH(mla::launch_zero_kv_padding((void*)k_nope, (void*)v_t, (void*)k_pe, B, H, T, Tp, dtype == MLA_F32 ? 4 : 2, s),
         "zero_kv_padding");
  mla::PrefillAttnArgs a{};
  a.q = q; a.kn = k_nope; a.vt = v_t; a.kpe = k_pe; a.mask = mask; a.out = out;
  a.B = B; a.T = T; a.Tp = Tp; a.H = H; a.scale = scale;
  if (dtype == MLA_F32) LAUNCH(mla::launch_prefill_attn_f32(a, s), "prefill_attn_f32");
  else LAUNCH(mla::launch_prefill_attn_bf16(a, s), "prefill_attn");
  return MLA_OK;
}

size_t mla_decode_attention_workspace_size(int32_t B, int32_t H, int32_t max_len) {
  if (B <= 0 || H <= 0 || max_len <= 0) return 0;
  const int ns = mla::decode_splits(B, H, max_len);
  if (ns == 1) return 256;
  return align256((size_t)ns * B * H * 512 * 2) + align256((size_t)ns * B * H * 4);
}

int mla_decode_attention(const void* q_lat, const void* cache, const int32_t* cache_len, void* o_lat, int32_t B,
                         int32_t H, int32_t max_len, float scale, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!q_lat || !cache || !cache_len || !o_lat) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (B <= 0 || H <= 0 || max_len <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  if (max_len > MAX_CACHE_LEN) return fail(MLA_INVALID_ARG, "max_len (%d) above %d", max_len, MAX_CACHE_LEN);
  if (H % 64) return fail(MLA_UNSUPPORTED, "H must be a multiple of 64");
  if (((uintptr_t)q_lat | (uintptr_t)cache | (uintptr_t)o_lat) & 15)
    return fail(MLA_UNSUPPORTED, "q_lat, cache and o_lat must be 16-byte aligned");
  const size_t need = mla_decode_attention_workspace_size(B, H, max_len);
  if (!ws || ws_bytes < need) return fail(MLA_INVALID_ARG, "workspace too small: need %zu bytes", need);
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  mla::DecodeAttnArgs a{};
  a.qlat = q_lat; a.cache = cache; a.cache_len = cache_len;
  a.R = B; a.H = H; a.max_len = max_len; a.scale = scale;
  a.splits = mla::decode_splits(B, H, max_len);
  Carver c(ws);
  if (a.splits == 1) {
    a.olat = o_lat;
  } else {
    a.part = c.take((size_t)a.splits * B * H * 512 * 2);
    a.lse = (float*)c.take((size_t)a.splits * B * H * 4);
  }
  LAUNCH(mla::launch_decode_attn(a, s), "decode_attn");
  if (a.splits > 1) LAUNCH(mla::launch_decode_combine(a.part, a.lse, a.splits, (int64_t)B * H, o_lat, s), "combine");
  return MLA_OK;
}

int mla_decode_attention_noalloc(const void* q_lat, const void* cache, const int32_t* cache_len, void* o_lat,
                                 int32_t B, int32_t H, int32_t max_len, float scale, void* stream) {
  g_err.clear();
  if (!q_lat || !cache || !cache_len || !o_lat) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (B <= 0 || H <= 0 || max_len <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  const size_t need = mla_decode_attention_workspace_size(B, H, max_len);
  if (need > mla::DECODE_SCRATCH_BYTES)
    return fail(MLA_INVALID_ARG, "needs %zu bytes of scratch, more than the %zu the library holds", need,
                mla::DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = mla::decode_scratch(&ws);
  if (e != hipSuccess) return fail(MLA_HIP_ERROR, "scratch lookup: %s", hipGetErrorString(e));
  const int rc = mla_decode_attention(q_lat, cache, cache_len, o_lat, B, H, max_len, scale, ws,
                                      mla::DECODE_SCRATCH_BYTES, stream);
  return rc;
}

int mla_rope_table(float* cos_tab, float* sin_tab, int32_t n_pos, float base, void* stream) {
  g_err.clear();
  if (!cos_tab || !sin_tab) return fail(MLA_INVALID_ARG, "NULL table");
  if (n_pos <= 0 || !(base > 1.f)) return fail(MLA_INVALID_ARG, "bad n_pos/base");
  LAUNCH(mla::launch_rope_table(cos_tab, sin_tab, n_pos, base, (hipStream_t)stream), "rope_table");
  return MLA_OK;
}

int mla_latent_e4m3_view(void* cache, int64_t rows, int64_t row_stride, int32_t kv_lora_rank, void* stream) {
  g_err.clear();
  if (!cache) return fail(MLA_INVALID_ARG, "NULL cache");
  if (rows < 0 || kv_lora_rank <= 0 || row_stride < kv_lora_rank) return fail(MLA_INVALID_ARG, "bad sizes");
  if (rows > (1LL << 40) / (kv_lora_rank / 128 > 0 ? kv_lora_rank / 128 : 1))
    return fail(MLA_INVALID_ARG, "too many rows");
  if (kv_lora_rank % 128) return fail(MLA_UNSUPPORTED, "kv_lora_rank must be a multiple of 128");
  if (row_stride % 8 || ((uintptr_t)cache & 15))
    return fail(MLA_UNSUPPORTED, "need row_stride % 8 == 0 and a 16-byte aligned cache");
  LAUNCH(mla::launch_latent_e4m3_view(cache, rows, row_stride, kv_lora_rank, (hipStream_t)stream),
         "latent_e4m3_view");
  return MLA_OK;
}

int mla_quant_e4m3_1x128(const void* a, int64_t lda, int32_t a_dtype, int32_t M, int32_t K, uint8_t* q, float* scales,
                         void* stream) {
  g_err.clear();
  if (!a || !q || !scales) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M < 0 || K <= 0 || lda < K) return fail(MLA_INVALID_ARG, "bad sizes");
  if (K % 128) return fail(MLA_UNSUPPORTED, "K must be a multiple of 128");
  if (a_dtype != MLA_F32 && a_dtype != MLA_BF16) return fail(MLA_UNSUPPORTED, "a_dtype must be F32 or BF16");
  if (lda % 8 || (((uintptr_t)a | (uintptr_t)q) & 15)) return fail(MLA_UNSUPPORTED, "need lda % 8 == 0 and 16-byte aligned a, q");
  LAUNCH(mla::launch_quant_1x128(a, lda, a_dtype, M, K, q, scales, (hipStream_t)stream), "quant_e4m3_1x128");
  return MLA_OK;
}

int mla_quant_e4m3_block128(const float* w, int32_t N, int32_t K, uint8_t* q, float* scales, void* stream) {
  g_err.clear();
  if (!w || !q || !scales) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (N <= 0 || K <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  LAUNCH(mla::launch_quant_block128(w, N, K, q, scales, (hipStream_t)stream), "quant_e4m3_block128");
  return MLA_OK;
}

int mla_topk_to_bitmask(const int32_t* topk_idx, int32_t B, int32_t T, int32_t topk, uint32_t* mask, void* stream) {
  g_err.clear();
  if (!topk_idx || !mask) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (B <= 0 || T <= 0 || topk <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  if (T > 65536 * 8) return fail(MLA_UNSUPPORTED, "T too large for the LDS row buffer");
  LAUNCH(mla::launch_topk_bitmask(topk_idx, B, T, topk, 0, T, mask, (hipStream_t)stream), "topk_to_bitmask");
  return MLA_OK;
}

size_t mla_swiglu_workspace_size(int32_t M, int32_t inter) {
  if (M <= 0 || inter <= 0) return 0;
  // [M, inter] gate and up products (the fused path uses the first as the product)
  const size_t one = (((size_t)M * inter * 2) + 255) & ~(size_t)255;
  return 3 * one;
}

int mla_swiglu_mlp(const void* x, int32_t M, int32_t hidden, int32_t inter, const void* w_gate, const void* w_up,
                   const void* w_down, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!x || !w_gate || !w_up || !w_down || !out || !ws) return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M <= 0 || hidden <= 0 || inter <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  if (hidden % 64 || inter % 64) return fail(MLA_UNSUPPORTED, "hidden and inter must be multiples of 64");
  if (((uintptr_t)x | (uintptr_t)w_gate | (uintptr_t)w_up | (uintptr_t)w_down | (uintptr_t)out) & 15)
    return fail(MLA_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (ws_bytes < mla_swiglu_workspace_size(M, inter)) return fail(MLA_INVALID_ARG, "workspace too small");
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const size_t one = (((size_t)M * inter * 2) + 255) & ~(size_t)255;
  uint16_t* h = (uint16_t*)ws;
  // h = silu(x . Wg^T) * (x . Wu^T): one GEMM over paired gate / up tiles with
  // the product in its epilogue, else two GEMMs and an elementwise pass
  mla::GemmArgs g = gemm_args(x, hidden, w_gate, hidden, h, inter, MLA_BF16, M, inter, hidden);
  g.W2 = w_up; g.ldw2 = hidden; g.epi = mla::EPI_SWIGLU;
  if (mla::gemm_bf16_swiglu_ok(g)) {
    LAUNCH(mla::launch_gemm_bf16(g, s), "gemm_bf16(gate|up + silu*mul)");
  } else {
    uint16_t* gt = (uint16_t*)((char*)ws + one);
    uint16_t* up = (uint16_t*)((char*)ws + 2 * one);
    LAUNCH(mla::launch_gemm_bf16(gemm_args(x, hidden, w_gate, hidden, gt, inter, MLA_BF16, M, inter, hidden), s),
           "gemm_bf16(gate)");
    LAUNCH(mla::launch_gemm_bf16(gemm_args(x, hidden, w_up, hidden, up, inter, MLA_BF16, M, inter, hidden), s),
           "gemm_bf16(up)");
    LAUNCH(mla::launch_silu_mul(gt, up, h, (int64_t)M * inter, s), "silu_mul");
  }
  // out = h . Wd^T
  LAUNCH(mla::launch_gemm_bf16(gemm_args(h, inter, w_down, inter, out, hidden, MLA_BF16, M, hidden, inter), s),
         "gemm_bf16(down)");
  return MLA_OK;
}

// split-K chunks of the e4m3 gate|up product when it has few output tiles
constexpr int SWIGLU_FP8_SPLITS = 2;

size_t mla_swiglu_e4m3_workspace_size(int32_t M, int32_t hidden, int32_t inter) {
  if (M <= 0 || hidden <= 0 || inter <= 0) return 0;
  Carver c(nullptr);
  c.take((size_t)M * hidden); c.take((size_t)M * (hidden / 128) * 4);   // x codes, scales
  c.take((size_t)SWIGLU_FP8_SPLITS * M * inter * 8);                    // [gate | up] fp32 partials
  c.take((size_t)M * inter); c.take((size_t)M * (inter / 128) * 4);     // h codes, scales
  return c.off;
}

int mla_swiglu_mlp_e4m3(const void* x, int32_t M, int32_t hidden, int32_t inter, const void* w_gate,
                        const float* gate_scale, const void* w_up, const float* up_scale, const void* w_down,
                        const float* down_scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!x || !w_gate || !w_up || !w_down || !gate_scale || !up_scale || !down_scale || !out || !ws)
    return fail(MLA_INVALID_ARG, "NULL pointer");
  if (M <= 0 || hidden <= 0 || inter <= 0) return fail(MLA_INVALID_ARG, "bad sizes");
  if (hidden % 128 || inter % 128) return fail(MLA_UNSUPPORTED, "hidden and inter must be multiples of 128");
  if (((uintptr_t)x | (uintptr_t)w_gate | (uintptr_t)w_up | (uintptr_t)w_down | (uintptr_t)out) & 15)
    return fail(MLA_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (ws_bytes < mla_swiglu_e4m3_workspace_size(M, hidden, inter)) return fail(MLA_INVALID_ARG, "workspace too small");
  if ((uintptr_t)ws & 255) return fail(MLA_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  Carver c(ws);
  uint8_t* xq = (uint8_t*)c.take((size_t)M * hidden);
  float* xs = (float*)c.take((size_t)M * (hidden / 128) * 4);
  float* gu = (float*)c.take((size_t)SWIGLU_FP8_SPLITS * M * inter * 8);
  uint8_t* hq = (uint8_t*)c.take((size_t)M * inter);
  float* hs = (float*)c.take((size_t)M * (inter / 128) * 4);
  // x in dynamic 1x128 groups, then [gate | up] in one product over the stacked weights
  LAUNCH(mla::launch_quant_1x128(x, hidden, MLA_BF16, M, hidden, xq, xs, s), "quant_e4m3_1x128(x)");
  mla::GemmFp8Args g{};
  g.A = xq; g.a_scale = xs; g.W = (const uint8_t*)w_gate; g.w_scale = gate_scale;
  g.W2 = (const uint8_t*)w_up; g.w2_scale = up_scale; g.n_split = inter;
  g.C = gu; g.ldc = 2 * inter; g.c_dtype = MLA_F32; g.M = M; g.N = 2 * inter; g.K = hidden; g.epi = mla::EPI_ROWMAJOR;
  // split-K when the output has too few 256 x 256 tiles for the chip (fp32 partials)
  const int tiles = ((M + 255) / 256) * ((2 * inter + 255) / 256);
  const int groups = hidden / 128;
  int splits = (tiles >= 192 || M < 256) ? 1 : SWIGLU_FP8_SPLITS;   // the big-tile path takes split-K
  if (splits > groups) splits = groups;
  const int per = (groups + splits - 1) / splits;
  if ((groups + per - 1) / per != splits) splits = 1;                // every chunk non-empty
  g.k_splits = splits; g.split_stride = (int64_t)M * 2 * inter;
  LAUNCH(mla::launch_gemm_fp8(g, s), "gemm_fp8(gate|up)");
  // h = silu(gate) * up, rounded to bf16 and quantised for the down projection in one pass
  LAUNCH(mla::launch_silu_mul_quant(gu, 2 * inter, splits, (int64_t)M * 2 * inter, M, inter, hq, hs, s),
         "silu_mul_quant");
  mla::GemmFp8Args d{};
  d.A = hq; d.a_scale = hs; d.W = (const uint8_t*)w_down; d.w_scale = down_scale; d.n_split = hidden;
  d.C = out; d.ldc = hidden; d.c_dtype = MLA_BF16; d.M = M; d.N = hidden; d.K = inter; d.epi = mla::EPI_ROWMAJOR;
  LAUNCH(mla::launch_gemm_fp8(d, s), "gemm_fp8(down)");
  return MLA_OK;
}

}  // extern "C"
