"""Thin ctypes binding of libmla.so (include/mla.h), same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers, streams as
the current torch stream's hipStream_t. Every computation runs in the HIP
library; if libmla.so is missing the first call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_INVALID_ARG, MLA_UNSUPPORTED, MLA_HIP_ERROR = 0, 1, 2, 3
MLA_F32, MLA_BF16, MLA_E4M3 = 0, 1, 2

_TORCH_DT = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16, torch.uint8: MLA_E4M3,
             torch.float8_e4m3fn: MLA_E4M3}

vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class MlaDims(ctypes.Structure):
    _fields_ = [("dim", i32), ("q_lora_rank", i32), ("kv_lora_rank", i32), ("n_heads", i32),
                ("qk_nope_head_dim", i32), ("qk_rope_head_dim", i32), ("v_head_dim", i32),
                ("softmax_scale", f32), ("rms_eps", f32)]


class MlaWeights(ctypes.Structure):
    _fields_ = [("weight_dtype", i32),
                ("wq_a", vp), ("wq_a_scale", vp), ("q_norm_w", vp),
                ("wq_b", vp), ("wq_b_scale", vp),
                ("wkv_a", vp), ("wkv_a_scale", vp), ("kv_norm_w", vp),
                ("wkv_b", vp), ("wkv_b_scale", vp),
                ("wo", vp), ("wo_scale", vp)]


_SIGS = {
    "mla_version": (ctypes.c_char_p, []),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_prefill_workspace_size": (sz, [ctypes.POINTER(MlaDims), i32, i32, i32, i32, i32]),
    "mla_prefill": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaWeights), vp, i32, i32, i32,
                                   vp, vp, i32, vp, i32, vp, vp, vp, sz, vp]),
    "mla_prefill_cached_workspace_size": (sz, [ctypes.POINTER(MlaDims), i32, i32, i32, i32, i32]),
    "mla_prefill_cached": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaWeights), vp, i32, i32, i32,
                                          vp, i32, vp, vp, i32, vp, i32, vp, vp, sz, vp]),
    "mla_decode_workspace_size": (sz, [ctypes.POINTER(MlaDims), i32, i32, i32]),
    "mla_decode_sparse": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaWeights), vp, i32, vp, i32, vp,
                                         vp, i32, vp, vp, i32, vp, vp, sz, vp]),
    "mla_prefill_absorbed_workspace_size": (sz, [ctypes.POINTER(MlaDims), i32, i32, i32]),
    "mla_prefill_absorbed": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaWeights), vp, i32, i32, vp,
                                            vp, i32, vp, i32, vp, vp, vp, sz, vp]),
    "mla_decode": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaWeights), vp, i32, vp, i32, vp,
                                  vp, vp, i32, vp, vp, sz, vp]),
    "gemm_bf16": (ctypes.c_int, [vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, vp]),
    "gemm_f32": (ctypes.c_int, [vp, i64, vp, i64, vp, i64, i32, i32, i32, vp]),
    "gemm_fp8_blockscaled": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp]),
    "rmsnorm_rope": (ctypes.c_int, [vp, i64, i32, i32, i32, vp, f32, i32, i32, i32, vp, vp, i32, vp, i32,
                                    vp, i64, i32, vp]),
    "mla_prefill_attention": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]),
    "mla_decode_attention_workspace_size": (sz, [i32, i32, i32]),
    "mla_decode_attention": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, f32, vp, sz, vp]),
    "mla_decode_attention_noalloc": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, f32, vp]),
    "mla_rope_table": (ctypes.c_int, [vp, vp, i32, f32, vp]),
    "gemm_decode_workspace_size": (sz, [i32, i32, i32, i32]),
    "gemm_bf16_decode": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, sz, vp]),
    "gemm_fp8_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, vp, sz, vp]),
    "mla_quant_e4m3_1x128": (ctypes.c_int, [vp, i64, i32, i32, i32, vp, vp, vp]),
    "mla_latent_e4m3_view": (ctypes.c_int, [vp, i64, i64, i32, vp]),
    "mla_quant_e4m3_block128": (ctypes.c_int, [vp, i32, i32, vp, vp, vp]),
    "mla_topk_to_bitmask": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
    "mla_swiglu_workspace_size": (sz, [i32, i32]),
    "mla_swiglu_mlp": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
    "mla_swiglu_e4m3_workspace_size": (sz, [i32, i32, i32]),
    "mla_swiglu_mlp_e4m3": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
}

_lib = None


def lib():
    """Load libmla.so (once) and declare the C signatures. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run head_latent_attention_fwd_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


class MlaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"mla status {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != MLA_OK:
        raise MlaError(rc, lib().mla_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}")


def mla_version():
    return lib().mla_version().decode()


def mla_last_error():
    return lib().mla_last_error().decode()


def make_dims(dim, q_lora_rank, kv_lora_rank, n_heads, softmax_scale=None, rms_eps=1e-6):
    return MlaDims(dim, q_lora_rank, kv_lora_rank, n_heads, 128, 64, 128,
                   (192.0 ** -0.5) if softmax_scale is None else softmax_scale, rms_eps)


def make_weights(w, weight_dtype):
    """w: dict of device tensors (wq_a, q_norm_w, wq_b, wkv_a, kv_norm_w, wkv_b, wo and, for
    e4m3, the *_scale tensors). The returned struct keeps references to them."""
    s = MlaWeights(weight_dtype, *[_ptr(w.get(n)) for n in (
        "wq_a", "wq_a_scale", "q_norm_w", "wq_b", "wq_b_scale", "wkv_a", "wkv_a_scale", "kv_norm_w",
        "wkv_b", "wkv_b_scale", "wo", "wo_scale")])
    s._keep = w
    return s


def mla_prefill_workspace_size(dims, weight_dtype, act_dtype, B, T, topk=0):
    return lib().mla_prefill_workspace_size(ctypes.byref(dims), weight_dtype, act_dtype, B, T, topk)


def mla_decode_workspace_size(dims, weight_dtype, B, max_len):
    return lib().mla_decode_workspace_size(ctypes.byref(dims), weight_dtype, B, max_len)


def workspace(nbytes, device="cuda"):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def mla_prefill(dims, weights, x, rope_cos, rope_sin, out, ws, topk_idx=None, kv_cache_out=None, stream=None):
    """x, out [B, T, dim] (bf16 or fp32); rope tables [>=T, 32] fp32; topk_idx [B, T, k] int32."""
    B, T, _ = x.shape
    for t, n in ((x, "x"), (out, "out"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin"), (ws, "ws")):
        _need(t, name=n)
    k = 0
    if topk_idx is not None:
        _need(topk_idx, torch.int32, "topk_idx")
        k = topk_idx.shape[-1]
    rc = lib().mla_prefill(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), _TORCH_DT[x.dtype], B, T,
                           _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], _ptr(topk_idx), k, _ptr(out),
                           _ptr(kv_cache_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return out


def mla_prefill_cached_workspace_size(dims, weight_dtype, B, T, start_pos, topk=0):
    return lib().mla_prefill_cached_workspace_size(ctypes.byref(dims), weight_dtype, B, T, start_pos, topk)


def mla_prefill_cached(dims, weights, x, start_pos, kv_cache, rope_cos, rope_sin, out, ws, topk_idx=None,
                       stream=None):
    """x, out [B, T, dim] bf16 at positions start_pos..start_pos+T-1; kv_cache [B, max_len, kv_lora+64]
    bf16 (rows < start_pos read, rows start_pos..start_pos+T-1 written); topk_idx [B, T, k] int32."""
    B, T, _ = x.shape
    for t, n in ((x, "x"), (kv_cache, "kv_cache"), (out, "out"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin"),
                 (ws, "ws")):
        _need(t, name=n)
    k = 0
    if topk_idx is not None:
        _need(topk_idx, torch.int32, "topk_idx")
        k = topk_idx.shape[-1]
    rc = lib().mla_prefill_cached(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T, int(start_pos),
                                  _ptr(kv_cache), kv_cache.shape[1], _ptr(rope_cos), _ptr(rope_sin),
                                  rope_cos.shape[0], _ptr(topk_idx), k, _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return out


def mla_decode(dims, weights, x, kv_cache, cache_len, rope_cos, rope_sin, out, ws, topk_idx=None, stream=None):
    """x, out [B, dim] bf16; kv_cache [B, max_len, kv_lora+64] bf16 (updated in place); cache_len [B] int32;
    topk_idx [B, k] int32 (optional): attend only the listed positions (mla_decode_sparse)."""
    B = x.shape[0]
    for t, n in ((x, "x"), (kv_cache, "kv_cache"), (out, "out"), (ws, "ws")):
        _need(t, name=n)
    _need(cache_len, torch.int32, "cache_len")
    if topk_idx is None:
        rc = lib().mla_decode(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, _ptr(kv_cache),
                              kv_cache.shape[1], _ptr(cache_len), _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0],
                              _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    else:
        _need(topk_idx, torch.int32, "topk_idx")
        rc = lib().mla_decode_sparse(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, _ptr(kv_cache),
                                     kv_cache.shape[1], _ptr(cache_len), _ptr(topk_idx), topk_idx.shape[-1],
                                     _ptr(rope_cos), _ptr(rope_sin), rope_cos.shape[0], _ptr(out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return out


def mla_prefill_absorbed_workspace_size(dims, B, T, topk):
    return lib().mla_prefill_absorbed_workspace_size(ctypes.byref(dims), B, T, topk)


def mla_prefill_absorbed(dims, weights, x, rope_cos, rope_sin, topk_idx, out, ws, kv_cache_out=None, stream=None):
    """Top-k prefill in the absorbed latent form. x, out [B, T, dim] bf16; topk_idx [B, T, k] int32."""
    B, T, _ = x.shape
    for t, n in ((x, "x"), (out, "out"), (ws, "ws")):
        _need(t, torch.bfloat16 if n != "ws" else None, n)
    _need(topk_idx, torch.int32, "topk_idx")
    rc = lib().mla_prefill_absorbed(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T, _ptr(rope_cos),
                                    _ptr(rope_sin), rope_cos.shape[0], _ptr(topk_idx), topk_idx.shape[-1], _ptr(out),
                                    _ptr(kv_cache_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return out


def gemm_bf16(A, W, C, stream=None):
    """C[M, N] = A[M, K] . W[N, K]^T; A, W bf16 (row stride may exceed K); C bf16 or fp32."""
    M, K = A.shape
    N = W.shape[0]
    rc = lib().gemm_bf16(_ptr(A), A.stride(0), _ptr(W), W.stride(0), _ptr(C), C.stride(0), _TORCH_DT[C.dtype],
                         M, N, K, _stream(stream))
    _check(rc)
    return C


def gemm_f32(A, W, C, stream=None):
    M, K = A.shape
    N = W.shape[0]
    rc = lib().gemm_f32(_ptr(A), A.stride(0), _ptr(W), W.stride(0), _ptr(C), C.stride(0), M, N, K, _stream(stream))
    _check(rc)
    return C


def gemm_fp8_blockscaled(Aq, a_scale, Wq, w_scale, C, stream=None):
    M, K = Aq.shape
    N = Wq.shape[0]
    for t, n in ((Aq, "Aq"), (a_scale, "a_scale"), (Wq, "Wq"), (w_scale, "w_scale")):
        _need(t, name=n)
    rc = lib().gemm_fp8_blockscaled(_ptr(Aq), _ptr(a_scale), _ptr(Wq), _ptr(w_scale), _ptr(C), C.stride(0),
                                    _TORCH_DT[C.dtype], M, N, K, _stream(stream))
    _check(rc)
    return C


def gemm_bf16_decode(A, W, C, ws=None, stream=None):
    """Decode-shaped C[M, N] = A[M, K] . W[N, K]^T (M <= 128), bf16, contiguous."""
    M, K = A.shape
    N = W.shape[0]
    if ws is None:
        ws = workspace(lib().gemm_decode_workspace_size(MLA_BF16, M, N, K), A.device)
    _check(lib().gemm_bf16_decode(_ptr(A), _ptr(W), _ptr(C), M, N, K, _ptr(ws), ws.numel(), _stream(stream)))
    return C


def gemm_fp8_decode(Aq, a_scale, Wq, w_scale, C, ws=None, stream=None):
    """Decode-shaped block-scaled e4m3 product (M <= 128), bf16 out."""
    M, K = Aq.shape
    N = Wq.shape[0]
    if ws is None:
        ws = workspace(lib().gemm_decode_workspace_size(MLA_E4M3, M, N, K), Aq.device)
    _check(lib().gemm_fp8_decode(_ptr(Aq), _ptr(a_scale), _ptr(Wq), _ptr(w_scale), _ptr(C), M, N, K, _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return C


def rmsnorm_rope(inp, out, norm_dim=0, gamma=None, eps=1e-6, rope_off=0, rope_heads=0, rope_stride=64,
                 rope_cos=None, rope_sin=None, pos=None, pos_period=1, stream=None):
    rows = inp.shape[0]
    rl = rope_cos.shape[0] if rope_cos is not None else 0
    rc = lib().rmsnorm_rope(_ptr(inp), inp.stride(0), _TORCH_DT[inp.dtype], rows, norm_dim, _ptr(gamma), eps,
                            rope_off, rope_heads, rope_stride, _ptr(rope_cos), _ptr(rope_sin), rl, _ptr(pos),
                            pos_period, _ptr(out), out.stride(0), _TORCH_DT[out.dtype], _stream(stream))
    _check(rc)
    return out


def pad64(T):
    return (T + 63) // 64 * 64


def mla_prefill_attention(q, k_nope, v_t, k_pe, out, B, T, H, scale=192.0 ** -0.5, mask=None, stream=None):
    """q [B*T, H*192]; k_nope [B, H, Tp, 128]; v_t [B, H, 128, Tp]; k_pe [B, Tp, 64]; out [B*T, H*128]
    (Tp = pad64(T); the padding keys are zeroed by the call)."""
    Tp = pad64(T)
    for t, shp, n in ((k_nope, (B, H, Tp, 128), "k_nope"), (v_t, (B, H, 128, Tp), "v_t"), (k_pe, (B, Tp, 64), "k_pe")):
        _need(t, q.dtype, n)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}")
    rc = lib().mla_prefill_attention(_ptr(q), _ptr(k_nope), _ptr(v_t), _ptr(k_pe), _ptr(mask), _ptr(out),
                                     _TORCH_DT[q.dtype], B, T, H, scale, _stream(stream))
    _check(rc)
    return out


def mla_decode_attention_workspace_size(B, H, max_len):
    return lib().mla_decode_attention_workspace_size(B, H, max_len)


def mla_decode_attention(q_lat, cache, cache_len, o_lat, ws=None, scale=192.0 ** -0.5, stream=None):
    """q_lat [B, H, 576], cache [B, max_len, 576], cache_len [B] int32, o_lat [B, H, 512];
    ws: workspace of mla_decode_attention_workspace_size bytes (allocated here when None)."""
    B, H, _ = q_lat.shape
    if ws is None:
        ws = workspace(mla_decode_attention_workspace_size(B, H, cache.shape[1]), q_lat.device)
    rc = lib().mla_decode_attention(_ptr(q_lat), _ptr(cache), _ptr(cache_len), _ptr(o_lat), B, H, cache.shape[1],
                                    scale, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return o_lat


def mla_decode_attention_noalloc(q_lat, cache, cache_len, o_lat, scale=192.0 ** -0.5, stream=None):
    """mla_decode_attention with the library's own scratch (no allocation anywhere in the call)."""
    B, H, _ = q_lat.shape
    rc = lib().mla_decode_attention_noalloc(_ptr(q_lat), _ptr(cache), _ptr(cache_len), _ptr(o_lat), B, H,
                                            cache.shape[1], scale, _stream(stream))
    _check(rc)
    return o_lat


def mla_rope_table(n_pos, base=10000.0, device="cuda", stream=None):
    c = torch.empty((n_pos, 32), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _check(lib().mla_rope_table(_ptr(c), _ptr(s), n_pos, base, _stream(stream)))
    return c, s


def mla_quant_e4m3_1x128(a, q=None, scales=None, stream=None):
    M, K = a.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=a.device) if q is None else q
    scales = torch.empty((M, K // 128), dtype=torch.float32, device=a.device) if scales is None else scales
    _check(lib().mla_quant_e4m3_1x128(_ptr(a), a.stride(0), _TORCH_DT[a.dtype], M, K, _ptr(q), _ptr(scales),
                                      _stream(stream)))
    return q, scales


def mla_latent_e4m3_view(cache, kv_lora_rank, stream=None):
    """In place: the latent part of every row of a [..., row] bf16 cache in its 1x128 e4m3 view."""
    _need(cache, torch.bfloat16, "cache")
    rows = cache.numel() // cache.shape[-1]
    _check(lib().mla_latent_e4m3_view(_ptr(cache), rows, cache.stride(-2), kv_lora_rank, _stream(stream)))
    return cache


def mla_quant_e4m3_block128(w, stream=None):
    _need(w, torch.float32, "w")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device=w.device)
    _check(lib().mla_quant_e4m3_block128(_ptr(w), N, K, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def mla_topk_to_bitmask(topk_idx, T=None, stream=None):
    _need(topk_idx, torch.int32, "topk_idx")
    B, Tq, k = topk_idx.shape
    T = Tq if T is None else T
    mask = torch.empty((B, Tq, (T + 31) // 32), dtype=torch.int32, device=topk_idx.device)
    _check(lib().mla_topk_to_bitmask(_ptr(topk_idx), B, T, k, _ptr(mask), _stream(stream)))
    return mask


def mla_swiglu_mlp(x, w_gate, w_up, w_down, out=None, ws=None, stream=None):
    """out = (silu(x w_gate^T) * (x w_up^T)) w_down^T, all bf16 on the device."""
    for t, n in ((x, "x"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _need(t, torch.bfloat16, n)
    M, hidden = x.shape
    inter = w_gate.shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    nbytes = lib().mla_swiglu_workspace_size(M, inter)
    if ws is None:
        ws = workspace(nbytes, x.device)
    _check(lib().mla_swiglu_mlp(_ptr(x), M, hidden, inter, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return out


def mla_swiglu_mlp_e4m3(x, gate, up, down, out=None, ws=None, stream=None):
    """SwiGLU MLP with e4m3 weights: gate, up, down are (codes uint8, scales fp32) pairs
    as mla_quant_e4m3_block128 returns them; x, out [M, hidden] bf16."""
    _need(x, torch.bfloat16, "x")
    for (c, sc), n in ((gate, "gate"), (up, "up"), (down, "down")):
        _need(c, torch.uint8, n)
        _need(sc, torch.float32, n + " scales")
    M, hidden = x.shape
    inter = gate[0].shape[0]
    if out is None:
        out = torch.empty((M, hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = workspace(lib().mla_swiglu_e4m3_workspace_size(M, hidden, inter), x.device)
    _check(lib().mla_swiglu_mlp_e4m3(_ptr(x), M, hidden, inter, _ptr(gate[0]), _ptr(gate[1]), _ptr(up[0]),
                                     _ptr(up[1]), _ptr(down[0]), _ptr(down[1]), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(stream)))
    return out
