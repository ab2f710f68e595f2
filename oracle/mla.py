"""Plain fp64 oracle of the multi-head latent attention (MLA) forward.

Test infrastructure only: imported by tests/, by smoke() in __graft_entry__.py
and by bench.py's cpu_baseline leg. The HIP library never imports, links or
calls anything here, and nothing here imports the library.

Every intermediate is kept in fp64; inputs arrive already rounded to the run
dtype (bf16/fp32 values are exact in fp64). numpy's matmul is the only library
primitive; attention is written per query row, over that row's live keys in
ascending order, straight from the definition.

Sources (the pages of the model atlas on MLA):
  [QC]  "Kimi K2 · Query compression" page: "Parameters" table, "Explanation",
        "Code" section (module init excerpt; query path excerpt).
  [OP]  "Kimi K2 · Output projection" page: the Delta_attn = o W_O formula,
        "Parameters" table, "Code" section (head flatten + o_proj excerpt).
  [DN]  "Kimi K2 · Down projection" page: formula y = h W_2, "Parameters"
        table, "Code" section (SwiGLU MLP; quantization_config).
  [SA]  "DeepSeek-V3.2-Exp · Sparse attention" page (prefill, empty cache):
        in/out shapes, "Explanation", "Code" section (MHA prefill excerpt).
  [DO]  "DeepSeek-V3.2-Exp · Output projection" page (decode, p=1000):
        shapes, "Parameters" table, "Code" section (MLA init excerpt).

Readings where the pages are silent:
  RMSNorm  y = gamma * x / sqrt(mean(x^2) + eps)      (only the class is named)
  RoPE     rotate-half over the 64 rotary dims: dim d pairs with d+32,
           theta_d = pos * base^(-d/32), base 10000    (no formula on the pages)
  positions 0..T-1 in prefill (empty cache); the decoded token sits at
           position cache_len and attends keys 0..cache_len inclusive.
"""
import numpy as np

NOPE, ROPE, VDIM = 128, 64, 128


def default_dims(dim, q_lora_rank, kv_lora_rank, n_heads, rms_eps=1e-6, rope_base=10000.0):
    """MLA dimensions. softmax_scale = qk_head_dim ** -0.5 with qk_head_dim =
    qk_nope + qk_rope = 192 ([DO] "Code": softmax_scale; the mscale branch is
    for extended contexts and is not taken)."""
    return dict(dim=dim, q_lora_rank=q_lora_rank, kv_lora_rank=kv_lora_rank,
                n_heads=n_heads, qk_nope_head_dim=NOPE, qk_rope_head_dim=ROPE,
                v_head_dim=VDIM, softmax_scale=float(NOPE + ROPE) ** -0.5,
                rms_eps=rms_eps, rope_base=rope_base)


def weight_shapes(d):
    """[out, in] shapes of the MLA weights ([QC] "Code": module init; [DO]
    "Code": MLA init; [OP] "The reference module holds the weight output by
    input"). No projection has a bias: the parameter tables leave no room."""
    H = d["n_heads"]
    qk = d["qk_nope_head_dim"] + d["qk_rope_head_dim"]
    return {
        "wq_a": (d["q_lora_rank"], d["dim"]),
        "q_norm_w": (d["q_lora_rank"],),
        "wq_b": (H * qk, d["q_lora_rank"]),
        "wkv_a": (d["kv_lora_rank"] + d["qk_rope_head_dim"], d["dim"]),
        "kv_norm_w": (d["kv_lora_rank"],),
        "wkv_b": (H * (d["qk_nope_head_dim"] + d["v_head_dim"]), d["kv_lora_rank"]),
        "wo": (d["dim"], H * d["v_head_dim"]),
    }


def swiglu_shapes(hidden, d_ff):
    """Shared-expert SwiGLU MLP weights ([DN] "Code": gate, up and down
    projections, all bias-free, [out, in])."""
    return {"gate": (d_ff, hidden), "up": (d_ff, hidden), "down": (hidden, d_ff)}


def n_params(shape):
    n = 1
    for s in shape:
        n *= s
    return n


# ----------------------------------------------------------------------------
# building blocks

def linear(x, w):
    """y = x . W^T for W held [out, in] ([OP] formula and layout note)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def rmsnorm(x, gamma, eps):
    """RMSNorm over the last axis (reading: y = gamma * x / sqrt(mean(x^2)+eps))."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope_angles(pos, base=10000.0, rope_dim=ROPE):
    """theta[..., d] = pos * base^(-2d/rope_dim), d = 0..rope_dim/2-1."""
    half = rope_dim // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / rope_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, base=10000.0):
    """Rotate-half RoPE on the last axis (64 dims): pair (d, d+32) is rotated by
    theta_d. x: [..., 64]; pos broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    th = rope_angles(pos, base, x.shape[-1])
    c, s = np.cos(th), np.sin(th)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax_over_live(z):
    """exp(z - max z) / sum exp(z - max z) over a 1-D or [H, n] array of live scores."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def live_keys(s, topk_row=None):
    """Keys a query at position s may attend ([SA] "Code": the selection mask
    is 0 at the indexer's picks and -inf elsewhere, and the causal mask is
    added on top): t <= s, and, with a selection, t among the picks. Ascending."""
    if topk_row is None:
        return np.arange(s + 1)
    sel = np.unique(np.asarray(topk_row)[np.asarray(topk_row) >= 0])
    return sel[sel <= s]


# ----------------------------------------------------------------------------
# projections shared by prefill and decode

def _proj(a, w, name, fp8):
    if fp8 is None:
        return linear(a, w[name])
    codes, scales = fp8[name]
    from .fp8 import linear_fp8
    return linear_fp8(a, codes, scales)


def quantise_weights(w):
    """Block-quantise every projection's fp32 master ([DN] quantization_config:
    e4m3, 128 x 128 weight blocks). Returns {name: (codes, scales)}."""
    from .fp8 import quant_weight_block128
    return {n: quant_weight_block128(w[n]) for n in ("wq_a", "wq_b", "wkv_a", "wkv_b", "wo")}


def query_path(x, w, d, pos, fp8=None):
    """Low-rank query path ([QC] "Code": q = q_b(q_a_norm(q_a(x))), viewed
    [.., H, 192] and split into a 128-dim non-rotated part and a 64-dim
    rotated part). Returns (q_nope [.., H, 128], q_pe [.., H, 64]) with RoPE
    applied to q_pe at the row's position."""
    H = d["n_heads"]
    cq = _proj(x, w, "wq_a", fp8)
    cqn = rmsnorm(cq, w["q_norm_w"], d["rms_eps"])
    q = _proj(cqn, w, "wq_b", fp8).reshape(x.shape[0], H, NOPE + ROPE)
    q_nope = q[:, :, :NOPE]
    q_pe = rope(q[:, :, NOPE:], np.asarray(pos)[:, None], d["rope_base"])
    return q_nope, q_pe


def latent_path(x, w, d, pos, fp8=None):
    """Joint KV down-projection ([QC] "Direct evidence": it emits the latent
    and the shared rotary key): kv = x . Wkv_a^T = [latent (kv_lora) | k_pe (64)];
    the latent gets RMSNorm, k_pe gets RoPE at the row's position. Returns the
    cache entry [.., kv_lora + 64] = [normalised latent | rotated k_pe]."""
    L = d["kv_lora_rank"]
    kv = _proj(x, w, "wkv_a", fp8)
    c = rmsnorm(kv[:, :L], w["kv_norm_w"], d["rms_eps"])
    k_pe = rope(kv[:, L:], np.asarray(pos), d["rope_base"])
    return np.concatenate([c, k_pe], axis=-1)


def up_project(c, w, d, fp8=None):
    """kv_b applied to normalised latents ([SA] "Code": viewed [.., H, 256]
    and split into k_nope (128) then v (128)). Returns (k_nope, v)."""
    H = d["n_heads"]
    u = _proj(c, w, "wkv_b", fp8).reshape(c.shape[0], H, NOPE + VDIM)
    return u[:, :, :NOPE], u[:, :, NOPE:]


def attend_row(q_nope, q_pe, k_nope, k_pe, v, live, scale):
    """One query row, all heads ([SA] "Code": scores = scale * q . k with
    k = [k_nope | shared k_pe], masked keys excluded, softmax over keys, then
    the probability-weighted sum of values).

    q_nope [H,128], q_pe [H,64]; k_nope [T,H,128], k_pe [T,64], v [T,H,128];
    live: ascending key indices. Returns (o [H,128], p [H, len(live)])."""
    kn = k_nope[live]                                   # [n, H, 128]
    z = np.einsum("hd,thd->ht", q_nope, kn) + (q_pe @ k_pe[live].T)
    z = z * scale
    p = softmax_over_live(z)                            # [H, n]
    o = np.einsum("ht,thd->hd", p, v[live])
    return o, p


# ----------------------------------------------------------------------------
# prefill

def mla_prefill(x, w, d, topk_idx=None, rows=None, fp8=False, return_aux=False):
    """MLA prefill forward with an empty cache ([SA] "Code" and shapes;
    [OP] head flatten + o_proj).

    x: [B, T, dim]; w: weights by name (bf16/fp32 values; with fp8=True the
    fp32 masters, which are block-quantised here first); topk_idx: optional
    [B, T, k] int selection (-1 = padding); rows: optional query positions to
    evaluate (all positions still produce keys and values).
    Returns out [B, len(rows), dim] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    fq = quantise_weights(w) if fp8 else None
    H = d["n_heads"]
    L = d["kv_lora_rank"]
    out = np.zeros((B, len(rows), d["dim"]))
    aux = {"p": [], "live": [], "cache": []}
    for b in range(B):
        pos_all = np.arange(T)
        entry = latent_path(x[b], w, d, pos_all, fq)          # [T, L+64]
        k_nope, v = up_project(entry[:, :L], w, d, fq)
        k_pe = entry[:, L:]
        q_nope, q_pe = query_path(x[b, rows], w, d, rows, fq)
        o = np.zeros((len(rows), H * VDIM))
        for i, s in enumerate(rows):
            live = live_keys(int(s), None if topk_idx is None else topk_idx[b, s])
            o_h, p = attend_row(q_nope[i], q_pe[i], k_nope, k_pe, v, live, d["softmax_scale"])
            o[i] = o_h.reshape(-1)
            if return_aux:
                aux["p"].append(p)
                aux["live"].append(live)
        out[b] = _proj(o, w, "wo", fq)
        if return_aux:
            aux["cache"].append(entry)
    return (out, aux) if return_aux else out


def mla_prefill_cached(x, w, d, cache, start_pos, topk_idx=None, rows=None, fp8=False):
    """Prefill of a chunk after start_pos cached tokens. The pages define the
    prefill with an empty cache ([SA] "Code", mode prefill) and the cache as
    the per-position [normalised latent | rotated k_pe] entries that decode
    scores ([SA] "Explanation"); read together, chunk token s sits at position
    P + s (P = start_pos), makes its entry like any prefill token, and attends
    keys 0..P+s: the cached entries followed by the chunk's own, all
    up-projected by kv_b as in prefill.

    x: [B, T, dim]; cache: [B, >= P, kv_lora + 64] entries of positions 0..P-1;
    topk_idx: optional [B, T, k] absolute key positions (-1 pads); rows:
    optional chunk rows to evaluate. Returns (out [B, len(rows), dim], the
    chunk's entries [B, T, kv_lora + 64])."""
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    P = int(start_pos)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    fq = quantise_weights(w) if fp8 else None
    H = d["n_heads"]
    L = d["kv_lora_rank"]
    out = np.zeros((B, len(rows), d["dim"]))
    entries = np.zeros((B, T, L + ROPE))
    for b in range(B):
        entries[b] = latent_path(x[b], w, d, P + np.arange(T), fq)
        C = np.concatenate([np.asarray(cache[b, :P], dtype=np.float64).reshape(P, L + ROPE), entries[b]], axis=0)
        k_nope, v = up_project(C[:, :L], w, d, fq)
        q_nope, q_pe = query_path(x[b, rows], w, d, P + rows, fq)
        o = np.zeros((len(rows), H * VDIM))
        for i, s in enumerate(rows):
            live = live_keys(P + int(s), None if topk_idx is None else topk_idx[b, s])
            o_h, _ = attend_row(q_nope[i], q_pe[i], k_nope, C[:, L:], v, live, d["softmax_scale"])
            o[i] = o_h.reshape(-1)
        out[b] = _proj(o, w, "wo", fq)
    return out, entries


# ----------------------------------------------------------------------------
# decode

def _decode_tokens(x, w, d, P, fp8=None):
    """Query parts and cache entries of the new tokens (row b at position P[b])."""
    q_nope, q_pe = query_path(x, w, d, P, fp8)
    entry = latent_path(x, w, d, P, fp8)
    return q_nope, q_pe, entry


def mla_decode(x, w, d, cache, cache_len, seqs=None, topk_idx=None, fp8=False):
    """Single-token decode, unabsorbed definition ([SA] "Explanation": one
    decoded token scores the cached latent; [DO] shapes [B,1,16384] -> [B,1,7168]).

    Per sequence b with P = cache_len[b]: the new token (position P) makes the
    entry [c | k_pe] and is appended at slot P; keys are slots 0..P (with
    topk_idx [B, k]: the listed ones among them, [SA] "Code" mask); every
    cached latent is up-projected by kv_b into per-head k_nope and v exactly
    as in prefill, then standard attention and wo.

    With fp8=True (w holds the fp32 masters, block-quantised here as in
    prefill, [DN] quantization_config) every Linear is the e4m3 block-scaled
    product with its input quantised in dynamic 1x128 groups, applied exactly
    as prefill applies it: q_a, kv_a and q_b to the new token, kv_b to every
    cached latent (and to the new one), wo to the flattened head outputs.
    Only live keys are up-projected (dead keys carry weight exactly 0).
    x: [B, dim]; cache: [B, max_len, kv_lora+64] values; cache_len: [B].
    Returns (out [len(seqs), dim], new_entry [len(seqs), kv_lora+64])."""
    x = np.asarray(x, dtype=np.float64)
    seqs = np.arange(x.shape[0]) if seqs is None else np.asarray(seqs)
    L = d["kv_lora_rank"]
    H = d["n_heads"]
    fq = quantise_weights(w) if fp8 else None
    P_all = np.asarray(cache_len)[seqs].astype(np.int64)
    q_nope, q_pe, entries = _decode_tokens(x[seqs], w, d, P_all, fq)
    o = np.zeros((len(seqs), H * VDIM))
    for i, b in enumerate(seqs):
        P = int(P_all[i])
        C = np.concatenate([np.asarray(cache[b, :P], dtype=np.float64), entries[i][None]], axis=0)
        C = C[live_keys(P, None if topk_idx is None else topk_idx[b])]
        k_nope, v = up_project(C[:, :L], w, d, fq)
        o_h, _ = attend_row(q_nope[i], q_pe[i], k_nope, C[:, L:], v, np.arange(C.shape[0]), d["softmax_scale"])
        o[i] = o_h.reshape(-1)
    return _proj(o, w, "wo", fq), entries


def mla_decode_absorbed(x, w, d, cache, cache_len, seqs=None, fp8=False, topk_idx=None):
    """Single-token decode with kv_b absorbed: mla_decode's result, reached by
    reassociating its products ([SA] "Explanation": the decoded token scores
    the cached latent directly). With W_UK_h = Wkv_b rows [256h, 256h+128) and
    W_UV_h = rows [256h+128, 256h+256), and c_t the latent kv_b receives:
      q_lat_h = W_UK_h^T q_nope_h                      (latent-space query)
      z[h, t] = scale * (q_lat_h . c_t + q_pe_h . k_pe_t)
      o_lat_h = sum_t softmax(z)[h, t] * c_t
      o_h     = W_UV_h o_lat_h
    With fp8=True the same reassociation of mla_decode(fp8=True): kv_b's
    product on a latent is the block-scaled e4m3 product, i.e. the product of
    the dequantised weight (codes times block scale) with the dequantised
    latent (its 1x128 codes times group scale). So W_UK and W_UV enter
    dequantised and c_t is the dequantised quantised latent, in the scores and
    in the values alike; the rotary key is not an input of kv_b and stays as
    cached. q_a, kv_a, q_b and wo stay e4m3 Linears.
    With topk_idx [B, k] only the listed slots among 0..P are keys.
    Returns (out, new_entry) like mla_decode."""
    x = np.asarray(x, dtype=np.float64)
    seqs = np.arange(x.shape[0]) if seqs is None else np.asarray(seqs)
    L = d["kv_lora_rank"]
    H = d["n_heads"]
    fq = quantise_weights(w) if fp8 else None
    if fp8:
        from .fp8 import dequant_weight, quant_dequant_act
        wkv_b = dequant_weight(*fq["wkv_b"])
    else:
        wkv_b = np.asarray(w["wkv_b"], dtype=np.float64)
    wkv_b = wkv_b.reshape(H, NOPE + VDIM, L)
    W_UK, W_UV = wkv_b[:, :NOPE, :], wkv_b[:, NOPE:, :]
    P_all = np.asarray(cache_len)[seqs].astype(np.int64)
    q_nope, q_pe, entries = _decode_tokens(x[seqs], w, d, P_all, fq)
    o = np.zeros((len(seqs), H * VDIM))
    for i, b in enumerate(seqs):
        P = int(P_all[i])
        C = np.concatenate([np.asarray(cache[b, :P], dtype=np.float64), entries[i][None]], axis=0)
        C = C[live_keys(P, None if topk_idx is None else topk_idx[b])]
        lat = quant_dequant_act(C[:, :L]) if fp8 else C[:, :L]
        q_lat = np.einsum("hi,hic->hc", q_nope[i], W_UK)           # [H, L]
        z = (q_lat @ lat.T + q_pe[i] @ C[:, L:].T) * d["softmax_scale"]
        p = softmax_over_live(z)                                  # [H, live keys]
        o_lat = p @ lat                                           # [H, L]
        o[i] = np.einsum("hjc,hc->hj", W_UV, o_lat).reshape(-1)   # [H*128]
    return _proj(o, w, "wo", fq), entries


# ----------------------------------------------------------------------------
# other pieces of the path, exposed for per-kernel checks

def rmsnorm_rope_rows(inp, norm_dim, gamma, eps, rope_off, rope_heads, rope_stride, pos, base):
    """Row-wise: RMSNorm over inp[:, :norm_dim] (if norm_dim > 0) and RoPE on
    rope_heads 64-dim slices at rope_off + h*rope_stride (if rope_heads > 0).
    Other elements pass through. Returns a new fp64 array."""
    out = np.array(inp, dtype=np.float64)
    if norm_dim > 0:
        out[:, :norm_dim] = rmsnorm(out[:, :norm_dim], gamma, eps)
    for h in range(rope_heads):
        o = rope_off + h * rope_stride
        out[:, o:o + ROPE] = rope(out[:, o:o + ROPE], np.asarray(pos), base)
    return out


def swiglu_mlp(x, wg, wu, wd, fp8=False):
    """Shared-expert SwiGLU MLP ([DN] "Direct evidence": down(silu(gate x) * up x)).
    With fp8=True the weights are fp32 masters, block-quantised here, and every
    Linear is the e4m3 block-scaled product of [DN] quantization_config."""
    if not fp8:
        g = linear(x, wg)
        return linear((g / (1.0 + np.exp(-g))) * linear(x, wu), wd)
    from .fp8 import linear_fp8, quant_weight_block128
    g = linear_fp8(x, *quant_weight_block128(wg))
    h = (g / (1.0 + np.exp(-g))) * linear_fp8(x, *quant_weight_block128(wu))
    return linear_fp8(h, *quant_weight_block128(wd))
