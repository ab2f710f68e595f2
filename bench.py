"""Benchmark of the MLA forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-kernels] [--workloads ...]

A step is one whole pass of the path over one batch of synthetic input that is
already resident in HBM: mla_prefill (x -> out) or mla_decode (x, cache -> out).
The headline is the largest single-GPU workload by algorithmic work: the
Kimi-K2-shaped prefill with e4m3 block-scaled weights (B = 4, T = 4096, 64
heads), in algorithmic TFLOP/s. The other workloads (bf16 prefill, sparse
DeepSeek-V3.2-Exp prefill, absorbed decode with bf16 and e4m3 weights, the
Kimi-K2 shared-expert MLP, chunked prefill, selected-key paths) are reported
beside it, each with the roofline of its dominant kernel. Every timed step is
preceded (outside its events) by a 1 GiB read, so weights, caches and
activations come from HBM, not from the 256 MB memory-side cache. Prints one
JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6, "fp8": 5033.2, "hbm": 8000.0}   # MI355X dense TFLOP/s and HBM GB/s
METRIC = "MLA prefill TFLOP/s + decode HBM GB/s (fraction of MI355X peak), 1 GPU"
HEADLINE = 2


# --------------------------------------------------------------------------
# algorithmic work

def live_pairs(cfg, topk_idx=None):
    B, T = cfg["B"], cfg["T"]
    if topk_idx is None:
        return B * T * (T + 1) // 2
    import numpy as np
    s = np.arange(T)[None, :, None]
    return int(((topk_idx >= 0) & (topk_idx <= s)).sum())


def gemm_shapes(cfg, M):
    """(M, N, K) of the four projection products of a prefill of M rows."""
    H, Dq, L, d = cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"]
    return {"q_a|kv_a": (M, Dq + L + 64, d), "q_b": (M, H * 192, Dq), "kv_b": (M, H * 256, L),
            "wo": (M, d, H * 128)}


def prefill_flops(cfg, topk_idx=None):
    M = cfg["B"] * cfg["T"]
    g = {k: 2 * m * n * kk for k, (m, n, kk) in gemm_shapes(cfg, M).items()}
    attn = 640 * cfg["n_heads"] * live_pairs(cfg, topk_idx)
    return sum(g.values()) + attn, g, attn


def decode_bytes(cfg):
    H, Dq, L, d, B, P = (cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"], cfg["B"],
                         cfg["cache_len"])
    n_w = (Dq + L + 64) * d + H * 192 * Dq + H * 256 * L + d * H * 128
    # bf16: 2 bytes a weight; e4m3: 1 byte plus one fp32 scale per 128 x 128 block
    w = n_w + 4 * n_w // (128 * 128) if cfg.get("weight") == "e4m3" else 2 * n_w
    keys = min(P + 1, cfg["topk"]) if cfg.get("topk") else P + 1   # a selection reads only its keys
    cache = 2 * B * keys * (L + 64)
    io = 2 * (2 * B * d + B * (L + 64)) + (4 * B * cfg["topk"] if cfg.get("topk") else 0)
    return w + cache + io, {"weights": w, "cache": cache, "io": io}


# --------------------------------------------------------------------------
# timing

class Flusher:
    """Reads 1 GiB so that the 256 MB memory-side cache and the L2s hold
    nothing of the step. A read, not a write: a write would leave dirty lines
    whose write-back then competes with the step's own reads."""

    def __init__(self):
        import torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def __call__(self):
        self.sink = self.buf.sum()


def timed_steps(fn, steps, warmup, flush):
    """Mean duration (s) of `steps` calls of fn, each bracketed by HIP events on
    the current stream (the one the library launches on) with a flush before
    it, outside its events; synchronised on both sides of the timed region."""
    import torch
    for _ in range(warmup):
        flush()
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps / 1e3


def timed_launches(fns, reps, warmup, flush):
    """Mean duration (s) of one kernel launch: each sample runs the calls in
    fns back to back between two HIP events, after a flush; fns work on
    distinct copies of the inputs (together larger than the memory-side
    cache), so every launch reads its operands from HBM, and the launch gap
    of the first call is shared by all of them."""
    import torch
    for _ in range(warmup):
        flush()
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for f in fns:
            f()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps / len(fns) / 1e3


def copies_for(nbytes):
    """Input copies whose total passes 512 MB (twice the memory-side cache)."""
    return max(1, min(8, -(-(512 << 20) // max(int(nbytes), 1))))


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "head_latent_attention_fwd_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(key, src_files):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current source of the kernel; else None."""
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json"))).get(key)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_hash") != source_hash(*src_files):
        return None
    return t.get("hbm_bytes_per_launch")


KERNEL_SOURCES = {"attention_prefill": ["attn_prefill.hip"], "attention_decode": ["attn_decode.hip"],
                  "gemm_bf16": ["gemm_bf16.hip"], "gemm_fp8": ["gemm_fp8.hip"], "skinny": ["gemm_skinny.hip"]}


# --------------------------------------------------------------------------
# workloads

def prefill_kernels(cfg, inp, run, flush, reps):
    """Per-launch kernel times from HIP events: each projection product and the
    attention launched through its building-block entry point with the
    workload's shapes (e4m3 operands quantised on the device), back to back on
    distinct input copies (see timed_launches)."""
    import torch
    from head_latent_attention_fwd_amd import api
    B, T, H = cfg["B"], cfg["T"], cfg["n_heads"]
    M = B * T
    dev, bf = "cuda", torch.bfloat16
    fp8 = cfg["weight"] == "e4m3"
    out = {}
    for name, (m, n, k) in gemm_shapes(cfg, M).items():
        C = torch.empty((m, n), device=dev, dtype=bf)
        fns = []
        for _ in range(copies_for((m * k + n * k) * (1 if fp8 else 2))):
            A = torch.randn((m, k), device=dev).to(bf)
            Wf = torch.randn((n, k), device=dev) / k ** 0.5
            if fp8:
                Aq, As = api.mla_quant_e4m3_1x128(A)
                Wq, Ws = api.mla_quant_e4m3_block128(Wf)
                fns.append(lambda Aq=Aq, As=As, Wq=Wq, Ws=Ws: api.gemm_fp8_blockscaled(Aq, As, Wq, Ws, C))
            else:
                W = Wf.to(bf)
                fns.append(lambda A=A, W=W: api.gemm_bf16(A, W, C))
            del A, Wf
        sec = timed_launches(fns, reps, 2, flush)
        flop = 2 * m * n * k
        peak = PEAK["fp8" if fp8 else "bf16"]
        out[("gemm_fp8_" if fp8 else "gemm_") + name] = {
            "us": sec * 1e6, "tflops": flop / sec / 1e12, "frac": flop / sec / 1e12 / peak, "flop": flop,
            "peak": peak, "src": "gemm_fp8" if fp8 else "gemm_bf16", "shape": [m, n, k], "launches_per_sample": len(fns)}
        del C, fns
        torch.cuda.empty_cache()
    Tp = api.pad64(T)
    o = torch.empty((M, H * 128), device=dev, dtype=bf)
    mask = None if inp["topk_idx"] is None else api.mla_topk_to_bitmask(run.topk)
    fns = []
    for _ in range(copies_for(2 * (M * H * 192 + 2 * B * H * Tp * 128 + B * Tp * 64))):
        q = torch.randn((M, H * 192), device=dev).to(bf)
        kn = torch.randn((B, H, Tp, 128), device=dev).to(bf)
        vt = torch.randn((B, H, 128, Tp), device=dev).to(bf)
        kp = torch.randn((B, Tp, 64), device=dev).to(bf)
        fns.append(lambda q=q, kn=kn, vt=vt, kp=kp: api.mla_prefill_attention(q, kn, vt, kp, o, B, T, H, mask=mask))
    sec = timed_launches(fns, reps, 2, flush)
    fl = 640 * H * live_pairs(cfg, inp["topk_idx"])
    out["attention"] = {"us": sec * 1e6, "tflops": fl / sec / 1e12, "frac": fl / sec / 1e12 / PEAK["bf16"],
                        "flop": fl, "peak": PEAK["bf16"], "src": "attention_prefill", "launches_per_sample": len(fns)}
    del o, fns
    torch.cuda.empty_cache()
    return out


def bench_prefill(cfg_index, steps, warmup, flush, kernels=False):
    import torch
    from head_latent_attention_fwd_amd import runner, synth
    cfg = synth.CONFIGS[cfg_index]
    inp = synth.gen_prefill(cfg, synth.seed_of(cfg_index))
    run = runner.Prefill(cfg, inp, keep_cache=False)
    flops, g, attn = prefill_flops(cfg, inp["topk_idx"])
    sec = timed_steps(run.run, steps, warmup, flush)
    res = {"workload": cfg["name"], "B": cfg["B"], "T": cfg["T"], "n_heads": cfg["n_heads"], "weights": cfg["weight"],
           "topk": cfg["topk"], "ms_per_step": sec * 1e3, "tflops": flops / sec / 1e12, "algorithmic_flop": flops}
    if cfg["weight"] == "e4m3":
        t_roof = sum(g.values()) / (PEAK["fp8"] * 1e12) + attn / (PEAK["bf16"] * 1e12)
        res["frac_of_mixed_roofline"] = t_roof / sec
    res["frac_of_bf16_peak"] = flops / sec / 1e12 / PEAK["bf16"]
    if kernels:
        res["kernels"] = prefill_kernels(cfg, inp, run, flush, max(5, steps // 2))
    del run
    torch.cuda.empty_cache()
    return res


def decode_kernels(cfg, run, parts, flush, reps):
    """The decode step's attention, and its three weight-streaming products
    through the decode-shaped GEMM entry points (the same kernels), timed alone
    (a product with K chunks includes the reduction of its partials)."""
    import torch
    from head_latent_attention_fwd_amd import api
    B, H, d, Dq, L = cfg["B"], cfg["n_heads"], cfg["dim"], cfg["q_lora_rank"], cfg["kv_lora_rank"]
    fp8 = cfg.get("weight") == "e4m3"
    out = {}
    ol = torch.empty((B, H, 512), device="cuda", dtype=torch.bfloat16)
    ws = api.workspace(api.mla_decode_attention_workspace_size(B, H, run.cache.shape[1]))
    fns = []
    for i in range(copies_for(parts["cache"])):
        ql = torch.randn((B, H, 576), device="cuda").to(torch.bfloat16)
        cache = run.cache if i == 0 else run.cache.clone()
        fns.append(lambda ql=ql, cache=cache: api.mla_decode_attention(ql, cache, run.cache_len, ol, ws=ws))
    s = timed_launches(fns, reps, 2, flush)
    out["attention"] = {"us": s * 1e6, "gbps": parts["cache"] / s / 1e9, "frac": parts["cache"] / s / 1e9 / PEAK["hbm"],
                        "bytes": parts["cache"], "peak": PEAK["hbm"], "src": "attention_decode",
                        "launches_per_sample": len(fns)}
    del fns
    for name, (n, k) in {"q_a|kv_a": (Dq + L + 64, d), "q_b": (H * 192, Dq), "wo": (d, H * 128)}.items():
        C = torch.empty((B, n), device="cuda", dtype=torch.bfloat16)
        if fp8:
            nbytes = n * k + 4 * (-(-n // 128)) * (k // 128) + B * k + 2 * B * n
            wsg = api.workspace(api.lib().gemm_decode_workspace_size(api.MLA_E4M3, B, n, k))
        else:
            nbytes = 2 * n * k + 2 * B * k + 2 * B * n
            wsg = api.workspace(api.lib().gemm_decode_workspace_size(api.MLA_BF16, B, n, k))
        fns = []
        for _ in range(copies_for(nbytes)):
            A = torch.randn((B, k), device="cuda").to(torch.bfloat16)
            Wf = torch.randn((n, k), device="cuda") / k ** 0.5
            if fp8:
                Aq, As = api.mla_quant_e4m3_1x128(A)
                Wq, Ws = api.mla_quant_e4m3_block128(Wf)
                fns.append(lambda Aq=Aq, As=As, Wq=Wq, Ws=Ws: api.gemm_fp8_decode(Aq, As, Wq, Ws, C, ws=wsg))
            else:
                W = Wf.to(torch.bfloat16)
                fns.append(lambda A=A, W=W: api.gemm_bf16_decode(A, W, C, ws=wsg))
            del Wf
        s = timed_launches(fns, reps, 2, flush)
        out[("gemm_fp8_" if fp8 else "gemm_") + name] = {
            "us": s * 1e6, "gbps": nbytes / s / 1e9, "frac": nbytes / s / 1e9 / PEAK["hbm"], "bytes": nbytes,
            "peak": PEAK["hbm"], "src": "skinny", "shape": [B, n, k], "launches_per_sample": len(fns)}
        del C, fns
    torch.cuda.empty_cache()
    return out


def bench_decode(cfg_index, steps, warmup, flush, kernels=False, weight="bf16", **over):
    import torch
    from head_latent_attention_fwd_amd import runner, synth
    cfg = dict(synth.CONFIGS[cfg_index], weight=weight, **over)
    inp = synth.gen_decode(cfg, synth.seed_of(cfg_index), max_len=cfg["cache_len"] + 1)
    run = runner.Decode(cfg, inp)
    nbytes, parts = decode_bytes(cfg)
    sec = timed_steps(run.run, steps, warmup, flush)   # cache slot P is rewritten identically each step
    name = cfg["name"] + ("_e4m3" if weight == "e4m3" else "") + (f"_top{cfg['topk']}" if cfg.get("topk") else "")
    res = {"workload": name, "B": cfg["B"], "cache_len": cfg["cache_len"], "n_heads": cfg["n_heads"],
           "weights": weight, "us_per_step": sec * 1e6, "gbps": nbytes / sec / 1e9,
           "frac_of_hbm": nbytes / sec / 1e9 / PEAK["hbm"], "algorithmic_bytes": nbytes, "bytes": parts}
    if kernels:
        res["kernels"] = decode_kernels(cfg, run, parts, flush, max(5, steps // 2))
    del run
    torch.cuda.empty_cache()
    return res


def bench_absorbed(cfg_index, steps, warmup, flush, T=None):
    """Top-k prefill computed in the absorbed latent form (gathered keys shared
    by all heads), on a DeepSeek-V3.2-Exp sparse shape; optionally also the
    dense-masked path at the same shape for the crossover."""
    import torch
    from head_latent_attention_fwd_amd import runner, synth
    cfg = dict(synth.CONFIGS[cfg_index])
    if T is not None:
        cfg["T"] = T
    inp = synth.gen_prefill(cfg, synth.seed_of(cfg_index))
    flops, g, attn = prefill_flops(cfg, inp["topk_idx"])
    run = runner.PrefillAbsorbed(cfg, inp)
    sec = timed_steps(run.run, steps, warmup, flush)
    res = {"workload": cfg["name"] + "_absorbed_gather", "B": cfg["B"], "T": cfg["T"], "n_heads": cfg["n_heads"],
           "topk": cfg["topk"], "ms_per_step": sec * 1e3, "tflops": flops / sec / 1e12,
           "frac_of_bf16_peak": flops / sec / 1e12 / PEAK["bf16"], "algorithmic_flop": flops}
    del run
    torch.cuda.empty_cache()
    if T is not None:   # the dense-masked path at the same shape
        dense = runner.Prefill(cfg, inp, keep_cache=False)
        res["dense_masked_ms_per_step"] = timed_steps(dense.run, steps, warmup, flush) * 1e3
        del dense
        torch.cuda.empty_cache()
    return res


def bench_chunk(steps, warmup, flush, start_pos=2048):
    """Kimi-K2 bf16 prefill of a 2048-token chunk after start_pos cached tokens
    (B = 1, H = 64): kv_b runs over all start_pos + 2048 latents."""
    import torch
    from head_latent_attention_fwd_amd import runner, synth
    cfg = synth.CONFIGS[1]
    inp = synth.gen_chunk(cfg, 6, start_pos)
    run = runner.PrefillCached(cfg, inp, start_pos)
    H, Dq, L, d, T = cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"], cfg["T"]
    pairs = T * start_pos + T * (T + 1) // 2
    flop = (2 * T * (Dq + L + 64) * d + 2 * T * H * 192 * Dq + 2 * (start_pos + T) * H * 256 * L
            + 2 * T * d * H * 128 + 640 * H * pairs)
    sec = timed_steps(run.run, steps, warmup, flush)
    res = {"workload": "kimi_k2_bf16_chunked_prefill", "B": 1, "T": T, "start_pos": start_pos, "n_heads": H,
           "ms_per_step": sec * 1e3, "tflops": flop / sec / 1e12, "frac_of_bf16_peak": flop / sec / 1e12 / PEAK["bf16"],
           "algorithmic_flop": flop}
    del run
    torch.cuda.empty_cache()
    return res


def bench_swiglu(steps, warmup, flush, M=2048, hidden=7168, inter=2048, e4m3=False):
    """Kimi-K2 shared-expert SwiGLU MLP over the prefill's 2048 tokens:
    out = (silu(x Wg^T) * (x Wu^T)) Wd^T, bf16 or e4m3 block-scaled weights."""
    import torch
    from head_latent_attention_fwd_amd import api
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((M, hidden), generator=g, device="cuda").to(torch.bfloat16)
    wg = torch.randn((inter, hidden), generator=g, device="cuda") / hidden ** 0.5
    wu = torch.randn((inter, hidden), generator=g, device="cuda") / hidden ** 0.5
    wd = torch.randn((hidden, inter), generator=g, device="cuda") / inter ** 0.5
    out = torch.empty((M, hidden), device="cuda", dtype=torch.bfloat16)
    flop = 2 * M * hidden * inter * 3
    if e4m3:
        q = [api.mla_quant_e4m3_block128(w) for w in (wg, wu, wd)]
        ws = api.workspace(api.lib().mla_swiglu_e4m3_workspace_size(M, hidden, inter))
        fn = lambda: api.mla_swiglu_mlp_e4m3(x, *q, out=out, ws=ws)
    else:
        wg, wu, wd = (w.to(torch.bfloat16) for w in (wg, wu, wd))
        ws = api.workspace(api.lib().mla_swiglu_workspace_size(M, inter))
        fn = lambda: api.mla_swiglu_mlp(x, wg, wu, wd, out=out, ws=ws)
    sec = timed_steps(fn, steps, warmup, flush)
    peak = PEAK["fp8"] if e4m3 else PEAK["bf16"]
    res = {"workload": "kimi_k2_shared_expert_mlp" + ("_e4m3" if e4m3 else ""), "M": M, "hidden": hidden,
           "inter": inter, "ms_per_step": sec * 1e3, "tflops": flop / sec / 1e12,
           ("frac_of_fp8_peak" if e4m3 else "frac_of_bf16_peak"): flop / sec / 1e12 / peak, "algorithmic_flop": flop}
    del x, wg, wu, wd, out, ws, fn
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------
# the oracle on the host cores

def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cores": threads}


def cpu_baseline(cfg_index, rows):
    """The fp64 oracle, as it stands, on a bounded sample of one workload.
    Prefill: keys and values of every position of the first sequence, then
    `rows` evenly spaced query rows through attention and o_proj (the rate is
    the sample's algorithmic flops over its time). Decode: `rows` sequences
    through the whole absorbed decode step (the rate is their algorithmic bytes
    over the time)."""
    import numpy as np
    from head_latent_attention_fwd_amd import synth
    from oracle import mla
    cfg = synth.CONFIGS[cfg_index]
    d = mla.default_dims(cfg["dim"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["n_heads"])
    H, Dq, L, dim = cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"]
    info = host_info()
    if cfg["mode"] == "decode":
        inp = synth.gen_decode(cfg, synth.seed_of(cfg_index), max_len=cfg["cache_len"] + 1)
        seqs = np.arange(rows)
        t0 = time.perf_counter()
        mla.mla_decode_absorbed(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], seqs=seqs)
        sec = time.perf_counter() - t0
        nbytes = decode_bytes(dict(cfg, B=rows))[0]
        return dict(info, value=nbytes / sec / 1e9, unit="GB/s", kind="oracle", seconds=sec, workload=cfg["name"],
                    sample=f"{cfg['name']}: {rows} of {cfg['B']} sequences through the absorbed decode step "
                           f"(fp64 numpy)")
    inp = synth.gen_prefill(dict(cfg, B=1), synth.seed_of(cfg_index))
    T = cfg["T"]
    sel = np.linspace(0, T - 1, rows).astype(int)
    topk = inp["topk_idx"]
    fp8 = cfg["weight"] == "e4m3"
    t0 = time.perf_counter()
    mla.mla_prefill(inp["x"], inp["w"], d, topk_idx=topk, rows=sel, fp8=fp8)
    sec = time.perf_counter() - t0
    pairs = int((sel + 1).sum()) if topk is None else int(sum(len(mla.live_keys(int(s), topk[0, s])) for s in sel))
    flop = (2 * T * (L + 64) * dim + 2 * T * H * 256 * L                       # keys/values, all positions
            + rows * (2 * Dq * dim + 2 * H * 192 * Dq + 2 * dim * H * 128)     # sampled rows
            + 640 * H * pairs)
    return dict(info, value=flop / sec / 1e12, unit="TFLOP/s", kind="oracle", seconds=sec, workload=cfg["name"],
                sample=f"{cfg['name']}: K/V for all {T} positions of one sequence, {rows} evenly spaced query rows "
                       f"through attention and o_proj (fp64 numpy" + (", e4m3 weights quantised on the host" if fp8
                                                                    else "") + ")")


# --------------------------------------------------------------------------

def roofline_of(res):
    """Roofline entry for the kernel that takes the most time in one workload."""
    ks = res["kernels"]
    dom = max(ks, key=lambda k: ks[k]["us"])
    k = ks[dom]
    src = KERNEL_SOURCES[k["src"]]
    common = {"workload": res["workload"], "kernel": dom, "peak": k["peak"], "frac": k["frac"],
              "us_per_launch": k["us"], "traffic": traffic_for(f"{res['workload']}:{dom}", src)}
    if "tflops" in k:
        return dict(common, bound="mfma", achieved=k["tflops"], unit="TFLOP/s", algorithmic_flop_per_launch=k["flop"])
    return dict(common, bound="hbm", achieved=k["gbps"], unit="GB/s", algorithmic_bytes_per_launch=k["bytes"])


WORKLOAD_HELP = ("2 Kimi-K2 prefill with e4m3 weights B4 T4096 (the headline); 1 the same in bf16, B1 T2048; "
                 "3 DeepSeek-V3.2-Exp top-2048 prefill T8192 (dense-masked); 4 DeepSeek-V3.2-Exp decode B128, 1000 "
                 "cached; 5 Kimi-K2 shared-expert SwiGLU MLP over 2048 tokens; 6 workload 1 as a chunk after 2048 "
                 "cached tokens; 7 workload 4 with e4m3 weights; 8 workload 3 in the absorbed gather form; 9 workload "
                 "4 over 4000 cached with a top-2048 selection; 10 the absorbed and dense-masked top-2048 prefill at "
                 "T16384; 11 workload 5 with e4m3 weights")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline legs")
    ap.add_argument("--workloads", default="2,1,3,4,5,6,7,8,9,11", help=WORKLOAD_HELP)
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel event breakdown")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (one GPU's share of a sharded "
              "layer is what it runs).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from head_latent_attention_fwd_amd import api
    api.lib()
    which = [int(x) for x in args.workloads.split(",") if x]
    kernels = not args.no_kernels
    flush = Flusher()
    results = {}
    for i in which:
        print(f"[bench] workload {i}", file=sys.stderr, flush=True)
        if i == 4:
            results[i] = bench_decode(4, args.steps, args.warmup, flush, kernels)
        elif i == 5:
            results[i] = bench_swiglu(args.steps, args.warmup, flush)
        elif i == 6:
            results[i] = bench_chunk(args.steps, args.warmup, flush)
        elif i == 7:
            results[i] = bench_decode(4, args.steps, args.warmup, flush, kernels, weight="e4m3")
        elif i == 8:
            results[i] = bench_absorbed(3, args.steps, args.warmup, flush)
        elif i == 9:
            results[i] = bench_decode(4, args.steps, args.warmup, flush, cache_len=4000, topk=2048)
        elif i == 10:
            results[i] = bench_absorbed(3, max(1, args.steps // 4), 1, flush, T=16384)
        elif i == 11:
            results[i] = bench_swiglu(args.steps, args.warmup, flush, e4m3=True)
        else:
            results[i] = bench_prefill(i, args.steps, args.warmup, flush, kernels and i in (1, 2, 3))
    head = results.get(HEADLINE, results[which[0]])
    fp8_head = head.get("weights") == "e4m3"
    line = {"metric": METRIC, "value": head.get("tflops", head.get("gbps")),
            "unit": "TFLOP/s" if "tflops" in head else "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head.get("ms_per_step", head.get("us_per_step", 0) / 1e3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "e4m3 projections + bf16 attention" if fp8_head else "bf16",
            "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights; 1 GiB read before each timed step)",
            "config": {k: head[k] for k in ("workload", "B", "T", "n_heads", "topk", "weights") if k in head}}
    if "frac_of_mixed_roofline" in head:
        line["frac_of_mixed_roofline"] = head["frac_of_mixed_roofline"]
    if "kernels" in head:
        line["roofline"] = roofline_of(head)
    line["rooflines"] = {r["workload"]: roofline_of(r) for r in results.values() if "kernels" in r}
    if 4 in results and "kernels" in results[4]:
        # The decode step's two largest kernels, both bound by HBM.
        for name, key in (("attention", "roofline_decode_attention"), ("gemm_wo", "roofline_decode_wo")):
            k = results[4]["kernels"][name]
            line[key] = {
                "workload": results[4]["workload"], "kernel": name, "bound": "hbm", "achieved": k["gbps"],
                "peak": PEAK["hbm"], "unit": "GB/s", "frac": k["frac"], "us_per_launch": k["us"],
                "algorithmic_bytes_per_launch": k["bytes"],
                "traffic": traffic_for(f"{results[4]['workload']}:{name}", KERNEL_SOURCES[k["src"]])}
    line["workloads"] = {str(k): v for k, v in results.items()}
    if not args.no_cpu:
        print("[bench] cpu baselines (oracle)", file=sys.stderr, flush=True)
        samples = {2: 24, 1: 256, 3: 32, 4: 64}
        base = {}
        for c, rows in samples.items():
            print(f"[bench] cpu baseline, workload {c}, {rows} sampled rows", file=sys.stderr, flush=True)
            base[str(c)] = cpu_baseline(c, rows)
        line["cpu_baseline"] = base[str(HEADLINE)]
        line["cpu_baselines"] = base
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
