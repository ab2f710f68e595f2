"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and rounds them to the run dtype; it
holds none of the attention arithmetic, so both the HIP path and the oracle can
consume its output. Recipe:

* numpy PCG64 (default_rng(seed)); every value is drawn in fp64 and rounded
  once (fp64 -> fp32 -> bf16, round-to-nearest-even) to the run dtype.
* x ~ N(0, 1); every weight W [out, in] ~ N(0, 1/in); RMSNorm gammas
  1 + 0.1 N(0, 1) (kept fp32).
* draw order: x, wq_a, q_norm_w, wq_b, wkv_a, kv_norm_w, wkv_b, wo, then the
  top-k selection (sparse prefill) or the cache (decode).
* top-k selection: query rows s < k keep every key 0..s; rows s >= k keep
  their own position plus k-1 distinct keys drawn uniformly from 0..s-1;
  stored ascending, int32, padded with -1.
* decode cache: slots 0..P-1 hold [latent | rope key]. The latent row is
  "N(0, 1), RMSNorm applied": z ~ N(0, 1), divided by sqrt(mean(z^2) + 1e-6)
  and multiplied by gamma_kv (the draw's distribution recipe, done in fp64
  before the one rounding to bf16). The rope key is N(0, 1), taken as already
  rotated (an isotropic Gaussian keeps its law under rotation). Slots >= P
  are 0. Chunked-prefill caches are drawn the same way.
* fp8 weights: the fp32 masters are returned; each side block-quantises them.
"""
import numpy as np

KV_ROPE = 64

# The five workloads: a tiny fp32 prefill, Kimi-K2-shaped prefills in bf16 and
# with fp8 weights, a DeepSeek-V3.2-Exp-shaped sparse prefill and a
# DeepSeek-V3.2-Exp-shaped absorbed decode.
CONFIGS = [
    dict(name="tiny_fp32_prefill", mode="prefill", B=1, T=64, dim=512, q_lora_rank=128,
         kv_lora_rank=64, n_heads=2, act="f32", weight="f32", topk=0),
    dict(name="kimi_k2_bf16_prefill", mode="prefill", B=1, T=2048, dim=7168, q_lora_rank=1536,
         kv_lora_rank=512, n_heads=64, act="bf16", weight="bf16", topk=0),
    dict(name="kimi_k2_fp8_prefill", mode="prefill", B=4, T=4096, dim=7168, q_lora_rank=1536,
         kv_lora_rank=512, n_heads=64, act="bf16", weight="e4m3", topk=0),
    dict(name="dsv32_sparse_prefill", mode="prefill", B=1, T=8192, dim=7168, q_lora_rank=1536,
         kv_lora_rank=512, n_heads=128, act="bf16", weight="bf16", topk=2048),
    dict(name="dsv32_absorbed_decode", mode="decode", B=128, cache_len=1000, dim=7168,
         q_lora_rank=1536, kv_lora_rank=512, n_heads=128, act="bf16", weight="bf16", topk=0),
]


def seed_of(config_index):
    return 1000 + config_index


def round_bf16(a):
    """fp64/fp32 array -> fp32 array holding the nearest bf16 values (ties to even)."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def round_to(a, dtype):
    if dtype == "bf16":
        return round_bf16(a)
    if dtype in ("f32", "e4m3"):
        return np.asarray(a, dtype=np.float32)
    raise ValueError(dtype)


def weight_shapes(cfg):
    H = cfg["n_heads"]
    return [
        ("wq_a", (cfg["q_lora_rank"], cfg["dim"])),
        ("q_norm_w", (cfg["q_lora_rank"],)),
        ("wq_b", (H * 192, cfg["q_lora_rank"])),
        ("wkv_a", (cfg["kv_lora_rank"] + KV_ROPE, cfg["dim"])),
        ("kv_norm_w", (cfg["kv_lora_rank"],)),
        ("wkv_b", (H * 256, cfg["kv_lora_rank"])),
        ("wo", (cfg["dim"], H * 128)),
    ]


def _draw_weights(rng, cfg):
    w = {}
    for name, shape in weight_shapes(cfg):
        if name.endswith("norm_w"):
            w[name] = (1.0 + 0.1 * rng.standard_normal(shape)).astype(np.float32)
        else:
            w[name] = round_to(rng.standard_normal(shape) / np.sqrt(shape[1]), cfg["weight"])
    return w


def draw_topk(rng, B, T, k, start=0):
    """Row s (at position start + s) keeps every earlier key if it has at most
    k, else itself plus k - 1 distinct earlier keys drawn uniformly."""
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for s in range(T):
            p = start + s
            if p < k:
                idx[b, s, :p + 1] = np.arange(p + 1)
            else:
                pick = rng.choice(p, k - 1, replace=False)
                idx[b, s] = np.sort(np.append(pick, p))
    return idx


def _normed_latents(rng, gamma, shape):
    """Cache latents per the decode workload: N(0, 1) rows scaled to unit root
    mean square (eps 1e-6 under the root) and multiplied by gamma."""
    z = rng.standard_normal(shape)
    return gamma * z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + 1e-6)


def make_cfg(index=None, **over):
    cfg = dict(CONFIGS[index]) if index is not None else {}
    cfg.update(over)
    return cfg


def gen_prefill(cfg, seed):
    """Inputs of one prefill: dict(x [B,T,dim] fp32 array, w {name: array}, topk_idx or None)."""
    rng = np.random.default_rng(seed)
    B, T = cfg["B"], cfg["T"]
    x = round_to(rng.standard_normal((B, T, cfg["dim"])), "f32" if cfg["act"] == "f32" else "bf16")
    w = _draw_weights(rng, cfg)
    topk = draw_topk(rng, B, T, cfg["topk"]) if cfg.get("topk") else None
    return dict(x=x, w=w, topk_idx=topk)


def gen_chunk(cfg, seed, start_pos, max_len=None):
    """Inputs of a prefill chunk after start_pos cached tokens: x [B,T,dim], w,
    cache [B,max_len,L+64] with rows < start_pos drawn like gen_decode's,
    topk_idx over absolute positions or None."""
    rng = np.random.default_rng(seed)
    B, T, L = cfg["B"], cfg["T"], cfg["kv_lora_rank"]
    max_len = max_len or (start_pos + T)
    x = round_to(rng.standard_normal((B, T, cfg["dim"])), "bf16")
    w = _draw_weights(rng, cfg)
    cache = np.zeros((B, max_len, L + KV_ROPE), dtype=np.float32)
    lat = _normed_latents(rng, w["kv_norm_w"].astype(np.float64), (B, start_pos, L))
    cache[:, :start_pos, :L] = round_to(lat, "bf16")
    cache[:, :start_pos, L:] = round_to(rng.standard_normal((B, start_pos, KV_ROPE)), "bf16")
    topk = draw_topk(rng, B, T, cfg["topk"], start_pos) if cfg.get("topk") else None
    return dict(x=x, w=w, cache=cache, topk_idx=topk)


def gen_decode(cfg, seed, max_len=None):
    """Inputs of one decode step: x [B,dim], w, cache [B,max_len,L+64] (slots >= P zero),
    cache_len [B] int32 (all P)."""
    rng = np.random.default_rng(seed)
    B, P = cfg["B"], cfg["cache_len"]
    L = cfg["kv_lora_rank"]
    max_len = max_len or (P + 1)
    x = round_to(rng.standard_normal((B, cfg["dim"])), "f32" if cfg["act"] == "f32" else "bf16")
    w = _draw_weights(rng, cfg)
    cache = np.zeros((B, max_len, L + KV_ROPE), dtype=np.float32)
    lat = _normed_latents(rng, w["kv_norm_w"].astype(np.float64), (B, P, L))
    cache[:, :P, :L] = round_to(lat, "bf16")
    cache[:, :P, L:] = round_to(rng.standard_normal((B, P, KV_ROPE)), "bf16")
    cache_len = np.full((B,), P, dtype=np.int32)
    topk = None
    if cfg.get("topk"):   # the new token at position P selects like a prefill row at P
        k = cfg["topk"]
        topk = np.full((B, k), -1, dtype=np.int32)
        for b in range(B):
            if P < k:
                topk[b, :P + 1] = np.arange(P + 1)
            else:
                topk[b] = np.sort(np.append(rng.choice(P, k - 1, replace=False), P))
    return dict(x=x, w=w, cache=cache, cache_len=cache_len, topk_idx=topk)
