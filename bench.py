"""Benchmark of the MLA forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workloads ...]

A step is one whole pass of the path over one batch of synthetic input that is
already resident in HBM: mla_prefill (x -> out) or mla_decode (x, cache -> out).
The headline value is the Kimi-K2-shaped bf16 prefill (B=1, T=2048, H=64) in
algorithmic TFLOP/s; the other workloads (fp8-weight prefill, sparse
DeepSeek-V3.2-Exp prefill, absorbed decode with bf16 and with e4m3 weights,
Kimi-K2 shared-expert MLP, chunked prefill over a 2048-token cache) are
reported beside it. Prints one
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


# --------------------------------------------------------------------------
# algorithmic work

def live_pairs(cfg, topk_idx=None):
    B, T = cfg["B"], cfg["T"]
    if topk_idx is None:
        return B * T * (T + 1) // 2
    import numpy as np
    s = np.arange(T)[None, :, None]
    return int(((topk_idx >= 0) & (topk_idx <= s)).sum())


def gemm_flops(cfg, M):
    H, Dq, L, d = cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"]
    return {"q_a|kv_a": 2 * M * (Dq + L + 64) * d, "q_b": 2 * M * H * 192 * Dq,
            "kv_b": 2 * M * H * 256 * L, "wo": 2 * M * d * H * 128}


def prefill_flops(cfg, topk_idx=None):
    M = cfg["B"] * cfg["T"]
    g = gemm_flops(cfg, M)
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
# timing helpers

def wall_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def event_avg(fn, reps, warmup=2, flush=None):
    """Average duration of fn's kernels from HIP events recorded on the current
    stream (the stream the library launches on). flush runs between reps,
    outside the timed events."""
    import torch
    for _ in range(warmup):
        fn()
    tot = 0.0
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        tot += a.elapsed_time(b)
    return tot / reps / 1e3   # seconds


class Flusher:
    """Reads 1 GiB so that the 256 MB MALL and the L2s hold nothing of the step.
    A read, not a write: a write would leave dirty lines whose write-back then
    competes with the step's own reads, which a model's other layers (mostly
    weight reads) would not cause."""

    def __init__(self):
        import torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def __call__(self):
        self.sink = self.buf.sum()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "head_latent_attention_fwd_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, src_files):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current source of the kernel; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(p)).get(kernel)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_hash") != source_hash(*src_files):
        return None
    return t.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# workloads

def bench_prefill(cfg_index, steps, warmup, kernels=False):
    import torch
    from head_latent_attention_fwd_amd import api, runner, synth
    cfg = synth.CONFIGS[cfg_index]
    inp = synth.gen_prefill(cfg, synth.seed_of(cfg_index))
    run = runner.Prefill(cfg, inp, keep_cache=False)
    flops, g, attn = prefill_flops(cfg, inp["topk_idx"])
    sec = wall_steps(run.run, steps, warmup)
    res = {"workload": cfg["name"], "B": cfg["B"], "T": cfg["T"], "n_heads": cfg["n_heads"], "weights": cfg["weight"],
           "topk": cfg["topk"], "ms_per_step": sec * 1e3, "tflops": flops / sec / 1e12,
           "algorithmic_flop": flops}
    fp8 = cfg["weight"] == "e4m3"
    if fp8:
        t_roof = sum(g.values()) / (PEAK["fp8"] * 1e12) + attn / (PEAK["bf16"] * 1e12)
        res["frac_of_mixed_roofline"] = t_roof / sec
        res["frac_of_bf16_peak"] = flops / sec / 1e12 / PEAK["bf16"]
    else:
        res["frac_of_bf16_peak"] = flops / sec / 1e12 / PEAK["bf16"]
    if kernels:
        res["kernels"] = prefill_kernel_breakdown(cfg, inp, run)
    del run
    torch.cuda.empty_cache()
    return res, inp


def prefill_kernel_breakdown(cfg, inp, run):
    """Per-step kernel times from HIP events, each step launched alone through
    its building-block entry point with the workload's shapes."""
    import torch
    from head_latent_attention_fwd_amd import api
    B, T, H, Dq, L, d = cfg["B"], cfg["T"], cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"]
    M = B * T
    dev = "cuda"
    bf = torch.bfloat16
    g = gemm_flops(cfg, M)
    out = {}
    shapes = {"q_a|kv_a": (M, Dq + L + 64, d), "q_b": (M, H * 192, Dq), "kv_b": (M, H * 256, L),
              "wo": (M, d, H * 128)}
    for name, (m, n, k) in shapes.items():
        A = torch.randn((m, k), device=dev).to(bf)
        W = (torch.randn((n, k), device=dev) / k ** 0.5).to(bf)
        C = torch.empty((m, n), device=dev, dtype=bf)
        sec = event_avg(lambda: api.gemm_bf16(A, W, C), 10)
        out["gemm_" + name] = {"us": sec * 1e6, "tflops": g[name] / sec / 1e12,
                               "frac": g[name] / sec / 1e12 / PEAK["bf16"], "flop": g[name]}
        del A, W, C
    Tp = api.pad64(T)
    q = torch.randn((M, H * 192), device=dev).to(bf)
    kn = torch.randn((B, H, Tp, 128), device=dev).to(bf)
    vt = torch.randn((B, H, 128, Tp), device=dev).to(bf)
    kp = torch.randn((B, Tp, 64), device=dev).to(bf)
    o = torch.empty((M, H * 128), device=dev, dtype=bf)
    mask = None
    if inp["topk_idx"] is not None:
        mask = api.mla_topk_to_bitmask(run.topk)
    pairs = live_pairs(cfg, inp["topk_idx"])
    sec = event_avg(lambda: api.mla_prefill_attention(q, kn, vt, kp, o, B, T, H, mask=mask), 10)
    fl = 640 * H * pairs
    out["attention"] = {"us": sec * 1e6, "tflops": fl / sec / 1e12, "frac": fl / sec / 1e12 / PEAK["bf16"],
                        "flop": fl}
    return out


def bench_decode(cfg_index, steps, warmup, kernels=False, weight="bf16", **over):
    import torch
    from head_latent_attention_fwd_amd import api, runner, synth
    cfg = dict(synth.CONFIGS[cfg_index], weight=weight, **over)
    inp = synth.gen_decode(cfg, synth.seed_of(cfg_index), max_len=cfg["cache_len"] + 1)
    run = runner.Decode(cfg, inp)
    nbytes, parts = decode_bytes(cfg)
    flush = Flusher()
    sec = event_avg(run.run, steps, warmup=warmup, flush=flush)   # cache slot P is rewritten identically each step
    res = {"workload": cfg["name"] + ("_e4m3" if weight == "e4m3" else "") + (f"_top{cfg['topk']}" if cfg.get("topk")
                                                                             else ""), "B": cfg["B"],
           "cache_len": cfg["cache_len"], "n_heads": cfg["n_heads"], "weights": weight, "us_per_step": sec * 1e6, "gbps": nbytes / sec / 1e9, "frac_of_hbm": nbytes / sec / 1e9 / PEAK["hbm"],
           "algorithmic_bytes": nbytes, "bytes": parts, "timing": "HIP events per step, 1 GiB read between steps (caches hold nothing of the step)"}
    if kernels:
        B, H = cfg["B"], cfg["n_heads"]
        ql = torch.randn((B, H, 576), device="cuda").to(torch.bfloat16)
        ol = torch.empty((B, H, 512), device="cuda", dtype=torch.bfloat16)
        s = event_avg(lambda: api.mla_decode_attention(ql, run.cache, run.cache_len, ol), 10, flush=flush)
        res["kernels"] = {"attention": {"us": s * 1e6, "gbps": parts["cache"] / s / 1e9,
                                        "frac": parts["cache"] / s / 1e9 / PEAK["hbm"], "bytes": parts["cache"]}}
    del run, flush
    torch.cuda.empty_cache()
    return res


def bench_absorbed(cfg_index, steps, warmup, T=None):
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
    sec = wall_steps(run.run, steps, warmup)
    res = {"workload": cfg["name"] + "_absorbed_gather", "B": cfg["B"], "T": cfg["T"], "n_heads": cfg["n_heads"],
           "topk": cfg["topk"], "ms_per_step": sec * 1e3, "tflops": flops / sec / 1e12,
           "frac_of_bf16_peak": flops / sec / 1e12 / PEAK["bf16"], "algorithmic_flop": flops}
    del run
    torch.cuda.empty_cache()
    if T is not None:   # the dense-masked path at the same shape
        dense = runner.Prefill(cfg, inp, keep_cache=False)
        sec_d = wall_steps(dense.run, steps, warmup)
        res["dense_masked_ms_per_step"] = sec_d * 1e3
        del dense
        torch.cuda.empty_cache()
    return res


def bench_chunk(steps, warmup, start_pos=2048):
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
    sec = wall_steps(run.run, steps, warmup)
    res = {"workload": "kimi_k2_bf16_chunked_prefill", "B": 1, "T": T, "start_pos": start_pos, "n_heads": H,
           "ms_per_step": sec * 1e3, "tflops": flop / sec / 1e12, "frac_of_bf16_peak": flop / sec / 1e12 / PEAK["bf16"],
           "algorithmic_flop": flop}
    del run
    torch.cuda.empty_cache()
    return res


def bench_swiglu(steps, warmup, M=2048, hidden=7168, inter=2048, e4m3=False):
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
    sec = wall_steps(fn, steps, warmup)
    peak = PEAK["fp8"] if e4m3 else PEAK["bf16"]
    res = {"workload": "kimi_k2_shared_expert_mlp" + ("_e4m3" if e4m3 else ""), "M": M, "hidden": hidden,
           "inter": inter, "ms_per_step": sec * 1e3, "tflops": flop / sec / 1e12,
           ("frac_of_fp8_peak" if e4m3 else "frac_of_bf16_peak"): flop / sec / 1e12 / peak, "algorithmic_flop": flop}
    del x, wg, wu, wd, out, ws, fn
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg_index, rows=256):
    """The fp64 oracle, as it stands, on a bounded sample of the prefill
    workload: keys/values for every position, then `rows` evenly spaced query
    rows through attention and o_proj."""
    import numpy as np
    from head_latent_attention_fwd_amd import synth
    from oracle import mla
    cfg = synth.CONFIGS[cfg_index]
    inp = synth.gen_prefill(cfg, synth.seed_of(cfg_index))
    d = mla.default_dims(cfg["dim"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["n_heads"])
    T, M = cfg["T"], cfg["B"] * cfg["T"]
    sel = np.linspace(0, T - 1, rows).astype(int)
    t0 = time.perf_counter()
    mla.mla_prefill(inp["x"], inp["w"], d, topk_idx=inp["topk_idx"], rows=sel)
    sec = time.perf_counter() - t0
    H, Dq, L, dim = cfg["n_heads"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["dim"]
    n = cfg["B"] * rows
    flop = (2 * M * (L + 64) * dim + 2 * M * H * 256 * L                       # keys/values, all rows
            + n * (2 * Dq * dim + 2 * H * 192 * Dq + 2 * dim * H * 128)        # sampled rows
            + 640 * H * cfg["B"] * int((sel + 1).sum()))
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": flop / sec / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": sec, "sample": f"{cfg['name']}: K/V for all {T} positions, {rows} evenly spaced query rows "
                                      f"through attention and o_proj (fp64 numpy)"}


def roofline_of(res):
    """Roofline entry for the kernel that takes the most time in one workload."""
    ks = res["kernels"]
    dom = max(ks, key=lambda k: ks[k]["us"])
    k = ks[dom]
    if "tflops" in k:
        src = ["attn_prefill.hip"] if dom == "attention" else ["gemm_bf16.hip"]
        return {"kernel": dom, "bound": "mfma", "achieved": k["tflops"], "peak": PEAK["bf16"], "unit": "TFLOP/s",
                "frac": k["frac"], "traffic": traffic_for(f"{res['workload']}:{dom}", src),
                "algorithmic_flop_per_launch": k["flop"], "us_per_launch": k["us"]}
    src = ["attn_decode.hip"] if dom == "attention" else ["gemm_skinny.hip"]
    return {"kernel": dom, "bound": "hbm", "achieved": k["gbps"], "peak": PEAK["hbm"], "unit": "GB/s",
            "frac": k["frac"], "traffic": traffic_for(f"{res['workload']}:{dom}", src),
            "algorithmic_bytes_per_launch": k.get("bytes"), "us_per_launch": k["us"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--workloads", default="1,2,3,4,5,6,7,8,9,11",
                    help="1 Kimi-K2 bf16 prefill B1 T2048 (the headline); 2 the same with e4m3 weights, B4 T4096; "
                         "3 DeepSeek-V3.2-Exp top-2048 prefill T8192 (dense-masked); 4 DeepSeek-V3.2-Exp decode "
                         "B128, 1000 cached; 5 Kimi-K2 shared-expert SwiGLU MLP over 2048 tokens; 6 workload 1 as "
                         "a chunk after 2048 cached tokens; 7 workload 4 with e4m3 weights; 8 workload 3 in the "
                         "absorbed gather form; 9 workload 4 over 4000 cached with a top-2048 selection; 10 the "
                         "absorbed and dense-masked top-2048 prefill at T16384; 11 workload 5 with e4m3 weights")
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
    results = {}
    head = None
    for i in which:
        print(f"[bench] workload {i}", file=sys.stderr, flush=True)
        if i == 4:
            results[i] = bench_decode(i, args.steps, args.warmup, kernels)
        elif i == 5:
            results[i] = bench_swiglu(args.steps, args.warmup)
        elif i == 6:
            results[i] = bench_chunk(args.steps, args.warmup)
        elif i == 7:
            results[i] = bench_decode(4, args.steps, args.warmup, weight="e4m3")
        elif i == 8:
            results[i] = bench_absorbed(3, args.steps, args.warmup)
        elif i == 9:
            results[i] = bench_decode(4, args.steps, args.warmup, cache_len=4000, topk=2048)
        elif i == 11:
            results[i] = bench_swiglu(args.steps, args.warmup, e4m3=True)
        elif i == 10:
            results[i] = bench_absorbed(3, max(1, args.steps // 4), 1, T=16384)
        else:
            results[i], _ = bench_prefill(i, args.steps, args.warmup, kernels and i == 1)
        if i == 1:
            head = results[i]
    if head is None:
        head = results[which[0]]
    line = {"metric": METRIC, "value": head.get("tflops", head.get("gbps")),
            "unit": "TFLOP/s" if "tflops" in head else "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head.get("ms_per_step", head.get("us_per_step", 0) / 1e3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
            "config": {k: head[k] for k in ("workload", "B", "T", "n_heads", "topk") if k in head}}
    if "kernels" in head:
        line["roofline"] = roofline_of(head)
    if 4 in results and results[4] is not head and "kernels" in results[4]:
        line["roofline_decode_attention"] = roofline_of(results[4])
    line["workloads"] = {str(k): v for k, v in results.items()}
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(1, rows=640)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
