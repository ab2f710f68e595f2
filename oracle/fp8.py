"""FP8 (OCP e4m3fn) codec and the 128-wide block quantisation, written from the
format definition. Test infrastructure only: imported by tests/, by smoke() in
__graft_entry__.py and by bench.py's cpu_baseline leg, never by the library.

What the pages fix (Kimi K2 "Down projection" page, config.json excerpt in its
"Code" section, and the "Direct evidence" note under it): weights are stored as
e4m3 with one scale per 128 x 128 block, and activations use a dynamic scheme.
The rest is the plainest reading the pages support:

* e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinity;
  S.1111.111 is NaN; largest finite magnitude 448; subnormal step 2^-9.
* encoding rounds to nearest, ties to the even mantissa, and saturates to +-448.
* a group's scale is amax / 448 in fp32 (so the group's largest element maps
  to +-448); an all-zero group gets scale 0 and codes 0.
* activations: one scale per row and per 128 consecutive elements along the
  reduction dimension; weights: one scale per 128 x 128 block of [out, in]
  (edge blocks partial, their max taken over the valid elements only).
* the quantiser's input is the activation tensor the Linear receives. The
  workload is a bf16 model ("bf16 in / fp32 accumulate", with fp8 weights as
  a variant of it), so that tensor holds bf16 values: the oracle rounds its
  fp64 activation to bf16 before quantising it. Scales are fp32 (the
  workload's "one fp32 scale per 128x128 block"); the quotient a / s of a
  bf16 value by an fp32 scale is taken in fp32, the precision both operands
  already have. A CPU test measures how far quantising the unrounded fp64
  activation instead would move a product of the fp8 workload's size.
"""
import numpy as np

E4M3_MAX = 448.0


def _magnitude_table():
    """Magnitudes of the 127 non-negative finite codes 0x00..0x7E, by definition."""
    mags = np.empty(127, dtype=np.float64)
    for code in range(127):
        e = code >> 3
        m = code & 7
        if e == 0:
            mags[code] = m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            mags[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return mags


_MAGS = _magnitude_table()


def e4m3_decode(codes):
    """uint8 codes -> float64 values (NaN for S.1111.111)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag_code = (codes & 0x7F).astype(np.int64)
    out = np.where(mag_code == 0x7F, np.nan, _MAGS[np.minimum(mag_code, 126)])
    return np.where(codes & 0x80, -out, out)


def e4m3_encode(values):
    """float values -> uint8 codes; round to nearest, ties to even, saturate.

    Finds the two representable magnitudes around |v| and keeps the nearer;
    on an exact tie keeps the one whose code (hence mantissa) is even.
    """
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # first mag >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(a == _MAGS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def group_scale_f32(amax):
    """Scale of a group whose largest magnitude is amax: amax/448, in fp32."""
    return (np.asarray(amax, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)


def _quantise_with_scale(vals, scale, quotient):
    """Codes of vals/scale; scale 0 gives code 0. quotient: 'f32' or 'f64'."""
    safe = np.where(scale == 0, np.float32(1), scale)
    if quotient == "f32":
        q = (vals.astype(np.float32) / safe.astype(np.float32)).astype(np.float32)
    else:
        q = vals.astype(np.float64) / safe.astype(np.float64)
    codes = e4m3_encode(q)
    return np.where(scale == 0, np.uint8(0), codes).astype(np.uint8)


def quant_act_1x128(a, quotient="f64"):
    """Dynamic activation quantisation: per row, per 128 elements along K.

    a: [M, K] real values (K % 128 == 0). Returns (codes uint8 [M, K],
    scales fp32 [M, K/128]). quotient selects the precision of a/scale:
    'f64' for the oracle's own fp64 activations, 'f32' when the input is
    already fp32/bf16 (the precision a GPU kernel divides in).
    """
    a = np.asarray(a)
    M, K = a.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    g = a.reshape(M, K // 128, 128)
    amax = np.abs(g).max(axis=2)
    if quotient == "f32":
        amax = amax.astype(np.float32)
    s = group_scale_f32(amax)                     # [M, K/128]
    codes = _quantise_with_scale(g, s[:, :, None], quotient)
    return codes.reshape(M, K), s


def quant_weight_block128(w):
    """Weight quantisation: one fp32 scale per 128 x 128 block of [N, K].

    w: fp32 master [N, K]. Edge blocks (N or K not a multiple of 128) take
    their max over the valid elements only. Division in fp32 (the weights
    are fp32). Returns (codes uint8 [N, K], scales fp32 [ceil(N/128), ceil(K/128)]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    nb, kb = -(-N // 128), -(-K // 128)
    scales = np.zeros((nb, kb), dtype=np.float32)
    codes = np.zeros((N, K), dtype=np.uint8)
    for i in range(nb):
        for j in range(kb):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            s = group_scale_f32(np.abs(blk).max())
            scales[i, j] = s
            codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = _quantise_with_scale(
                blk, np.full(blk.shape, s, dtype=np.float32), "f32")
    return codes, scales


def fp8_gemm(a_codes, a_scales, w_codes, w_scales):
    """Block-scaled product, accumulated in fp64 (Kimi K2 "Down projection"
    page, quantization_config): for each output
    y[m, n] = sum_g s_a[m, g] * s_w[n // 128, g] * sum_{k in group g} dec(a_q[m, k]) * dec(w_q[n, k]).
    The inner sums are exact in fp64 (products of two e4m3 values)."""
    M, K = a_codes.shape
    N = w_codes.shape[0]
    A = e4m3_decode(a_codes)                       # [M, K]
    W = e4m3_decode(w_codes)                       # [N, K]
    y = np.zeros((M, N), dtype=np.float64)
    sw_rows = w_scales[np.arange(N) // 128].astype(np.float64)   # [N, G]
    for g in range(K // 128):
        part = A[:, g * 128:(g + 1) * 128] @ W[:, g * 128:(g + 1) * 128].T
        y += part * a_scales[:, g:g + 1].astype(np.float64) * sw_rows[None, :, g]
    return y


def round_bf16(x):
    """Nearest bfloat16 value of each fp64 element (8 significant bits, ties to
    even), computed directly from fp64: x = m * 2^e with 0.5 <= |m| < 1, keep
    rint(m * 256) / 256. Values here never reach the bf16 subnormal range."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def dequant_weight(w_codes, w_scales):
    """Value the block-scaled weight stands for: codes times their block's scale."""
    N, K = w_codes.shape
    s = np.repeat(np.repeat(np.asarray(w_scales, dtype=np.float64), 128, 0), 128, 1)[:N, :K]
    return e4m3_decode(w_codes) * s


def quant_dequant_act(a):
    """Value an activation stands for after the dynamic 1x128 quantisation that
    linear_fp8 applies to its input (bf16 activation, fp32 quotient): each
    code times its group's scale. fp8_gemm of these codes equals the product
    of this array with the dequantised weight, so a reassociated product (an
    absorbed weight) sees the same operand."""
    codes, scales = quant_act_1x128(round_bf16(a).astype(np.float32), "f32")
    return e4m3_decode(codes) * np.repeat(scales.astype(np.float64), 128, axis=1)


def linear_fp8(a, w_codes, w_scales):
    """y = a . W^T with e4m3 operands. The activation is held in bf16 (the
    workload's activation dtype), quantised in dynamic 1x128 groups along K
    with the quotient in fp32, then the block-scaled product in fp64."""
    a_codes, a_scales = quant_act_1x128(round_bf16(a).astype(np.float32), "f32")
    return fp8_gemm(a_codes, a_scales, w_codes, w_scales)
