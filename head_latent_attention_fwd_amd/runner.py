"""Device-side setup around the C ABI: uploads weights and inputs, allocates
outputs and the workspace once, and runs a whole prefill or decode step.

Used by the tests, smoke() and bench.py. Only memory management lives here;
every step of the path runs in libmla.so (fp8 weights are block-quantised on
the device by mla_quant_e4m3_block128).
"""
import numpy as np
import torch

from . import api

_ACT = {"f32": torch.float32, "bf16": torch.bfloat16}
_WDT = {"f32": api.MLA_F32, "bf16": api.MLA_BF16, "e4m3": api.MLA_E4M3}
PROJ = ("wq_a", "wq_b", "wkv_a", "wkv_b", "wo")


def to_dev(a, dtype, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dtype)


def device_weights(w_np, weight, device="cuda"):
    """Weights as device tensors in the path's format. e4m3: the fp32 masters are
    uploaded and block-quantised by the library (codes as uint8 + fp32 scales)."""
    out = {"q_norm_w": to_dev(w_np["q_norm_w"], torch.float32, device),
           "kv_norm_w": to_dev(w_np["kv_norm_w"], torch.float32, device)}
    for n in PROJ:
        if weight == "e4m3":
            master = to_dev(w_np[n], torch.float32, device)
            out[n], out[n + "_scale"] = api.mla_quant_e4m3_block128(master)
            del master
        else:
            out[n] = to_dev(w_np[n], _ACT[weight], device)
    return out


def dims_of(cfg):
    return api.make_dims(cfg["dim"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["n_heads"])


class Prefill:
    """One MLA prefill (empty cache) with preallocated buffers."""

    def __init__(self, cfg, inp, device="cuda", keep_cache=True):
        self.cfg = cfg
        B, T = cfg["B"], cfg["T"]
        act = _ACT[cfg["act"]]
        self.dims = dims_of(cfg)
        self.wdt = _WDT[cfg["weight"]]
        self.x = to_dev(inp["x"], act, device)
        self.w = device_weights(inp["w"], cfg["weight"], device)
        self.weights = api.make_weights(self.w, self.wdt)
        self.cos, self.sin = api.mla_rope_table(T, device=device)
        self.topk = None if inp.get("topk_idx") is None else to_dev(inp["topk_idx"], torch.int32, device)
        self.out = torch.empty_like(self.x)
        self.kv_cache = (torch.empty((B, T, cfg["kv_lora_rank"] + 64), dtype=act, device=device)
                         if keep_cache else None)
        k = 0 if self.topk is None else self.topk.shape[-1]
        self.ws = api.workspace(api.mla_prefill_workspace_size(self.dims, self.wdt, api._TORCH_DT[act], B, T, k),
                                device)

    def run(self, stream=None):
        return api.mla_prefill(self.dims, self.weights, self.x, self.cos, self.sin, self.out, self.ws,
                               topk_idx=self.topk, kv_cache_out=self.kv_cache, stream=stream)


class PrefillCached:
    """One prefill chunk of T tokens after start_pos cached ones, over a
    [B, max_len, kv_lora + 64] bf16 cache (rows < start_pos given)."""

    def __init__(self, cfg, inp, start_pos, device="cuda"):
        self.cfg = cfg
        B, T = cfg["B"], cfg["T"]
        self.start_pos = start_pos
        self.dims = dims_of(cfg)
        self.wdt = _WDT[cfg["weight"]]
        self.x = to_dev(inp["x"], torch.bfloat16, device)
        self.w = device_weights(inp["w"], cfg["weight"], device)
        self.weights = api.make_weights(self.w, self.wdt)
        self.cache = to_dev(inp["cache"], torch.bfloat16, device)
        self.cos, self.sin = api.mla_rope_table(self.cache.shape[1], device=device)
        self.topk = None if inp.get("topk_idx") is None else to_dev(inp["topk_idx"], torch.int32, device)
        self.out = torch.empty_like(self.x)
        k = 0 if self.topk is None else self.topk.shape[-1]
        self.ws = api.workspace(api.mla_prefill_cached_workspace_size(self.dims, self.wdt, B, T, start_pos, k),
                                device)

    def run(self, stream=None):
        return api.mla_prefill_cached(self.dims, self.weights, self.x, self.start_pos, self.cache, self.cos,
                                      self.sin, self.out, self.ws, topk_idx=self.topk, stream=stream)


class Decode:
    """One single-token MLA decode step over a [B, max_len, 576] bf16 cache."""

    def __init__(self, cfg, inp, device="cuda"):
        self.cfg = cfg
        B = cfg["B"]
        self.dims = dims_of(cfg)
        self.wdt = _WDT[cfg.get("weight", "bf16")]
        self.x = to_dev(inp["x"], torch.bfloat16, device)
        self.w = device_weights(inp["w"], cfg.get("weight", "bf16"), device)
        self.weights = api.make_weights(self.w, self.wdt)
        self.cache0 = to_dev(inp["cache"], torch.bfloat16, device)
        if self.wdt == api.MLA_E4M3:   # with e4m3 weights the cache holds each latent in its e4m3 view
            api.mla_latent_e4m3_view(self.cache0, cfg["kv_lora_rank"])
        self.cache = self.cache0.clone()
        self.cache_len = to_dev(inp["cache_len"], torch.int32, device)
        max_len = self.cache.shape[1]
        self.cos, self.sin = api.mla_rope_table(max_len, device=device)
        self.out = torch.empty((B, cfg["dim"]), dtype=torch.bfloat16, device=device)
        self.ws = api.workspace(api.mla_decode_workspace_size(self.dims, self.wdt, B, max_len), device)
        self.topk = None if inp.get("topk_idx") is None else to_dev(inp["topk_idx"], torch.int32, device)

    def run(self, stream=None):
        return api.mla_decode(self.dims, self.weights, self.x, self.cache, self.cache_len, self.cos, self.sin,
                              self.out, self.ws, topk_idx=self.topk, stream=stream)


class PrefillAbsorbed:
    """One top-k prefill in the absorbed latent form (bf16)."""

    def __init__(self, cfg, inp, device="cuda"):
        self.cfg = cfg
        B, T = cfg["B"], cfg["T"]
        self.dims = dims_of(cfg)
        self.x = to_dev(inp["x"], torch.bfloat16, device)
        self.w = device_weights(inp["w"], "bf16", device)
        self.weights = api.make_weights(self.w, api.MLA_BF16)
        self.cos, self.sin = api.mla_rope_table(T, device=device)
        self.topk = to_dev(inp["topk_idx"], torch.int32, device)
        self.out = torch.empty_like(self.x)
        self.kv_cache = torch.empty((B, T, cfg["kv_lora_rank"] + 64), dtype=torch.bfloat16, device=device)
        self.ws = api.workspace(api.mla_prefill_absorbed_workspace_size(self.dims, B, T, self.topk.shape[-1]), device)

    def run(self, stream=None):
        return api.mla_prefill_absorbed(self.dims, self.weights, self.x, self.cos, self.sin, self.topk, self.out,
                                        self.ws, kv_cache_out=self.kv_cache, stream=stream)
