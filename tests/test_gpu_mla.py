"""End-to-end parity of mla_prefill / mla_decode against the fp64 oracle (GPU).

Small cases are compared element by element; the full-size workloads are
compared on sampled query rows (every position still feeds keys and values)
or on every decoded sequence.
"""
import numpy as np
import pytest
import torch

from head_latent_attention_fwd_amd import api, runner, synth
from oracle import mla
from oracle.fp8 import quant_weight_block128

from helpers import BF16_TOL, F32_TOL, FP8_TOL, assert_parity, config, e4m3_entries, oracle_dims, small_cfg

pytestmark = pytest.mark.gpu


def _prefill(cfg, seed):
    inp = synth.gen_prefill(cfg, seed)
    run = runner.Prefill(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    return inp, run


def _check_prefill(cfg, seed, rows=None, batches=None, tol=BF16_TOL, cos=0.9999):
    inp, run = _prefill(cfg, seed)
    got = run.out.float().cpu().numpy()
    d = oracle_dims(cfg)
    b_sel = np.arange(cfg["B"]) if batches is None else np.asarray(batches)
    topk = None if inp["topk_idx"] is None else inp["topk_idx"][b_sel]
    ref = mla.mla_prefill(inp["x"][b_sel], inp["w"], d, topk_idx=topk, rows=rows, fp8=cfg["weight"] == "e4m3")
    g = got[b_sel] if rows is None else got[b_sel][:, rows]
    assert_parity(g, ref, tol=tol, cos=cos, what=cfg["name"])
    return inp, run


def test_prefill_tiny_fp32_config():
    _check_prefill(config(0), synth.seed_of(0), tol=F32_TOL, cos=0.999999)


def test_prefill_small_bf16_dense():
    inp, run = _check_prefill(small_cfg(), 21)
    # the cache entries [c | k_pe] written by prefill
    d = oracle_dims(small_cfg())
    entry = mla.latent_path(inp["x"][1], inp["w"], d, np.arange(200))
    assert_parity(run.kv_cache[1].float().cpu().numpy(), entry, what="kv_cache_out")


def test_prefill_small_bf16_topk_ragged():
    _check_prefill(small_cfg(T=333, B=1, topk=40, n_heads=2), 22)


def test_prefill_small_fp32_topk():
    _check_prefill(small_cfg(T=70, B=2, topk=16, act="f32", weight="f32", dim=256), 23, tol=F32_TOL,
                   cos=0.999999)


def test_prefill_small_fp8():
    _check_prefill(small_cfg(T=160, dim=1024, q_lora_rank=512, kv_lora_rank=512, n_heads=4, weight="e4m3"), 24,
                   tol=FP8_TOL, cos=0.999)


def test_prefill_ragged_batches_cross_store_groups():
    # T = 261: the second sequence starts inside a group of 8 token rows, so
    # kv_b's v^T stores take both the 16-byte and the element-wise path
    _check_prefill(small_cfg(T=261, B=2, n_heads=2), 27)
    _check_prefill(small_cfg(T=261, B=2, dim=1024, q_lora_rank=512, kv_lora_rank=512, n_heads=2, weight="e4m3"), 28,
                   tol=FP8_TOL, cos=0.999)


def test_prefill_single_token_and_tiny_T():
    _check_prefill(small_cfg(T=1, B=3), 25)
    _check_prefill(small_cfg(T=2, B=1, topk=1), 26)


def _sample_rows(T, rng, n=10):
    fixed = [0, 1, 63, 64, 127, 128, T // 2, T - 1]
    return np.unique(np.concatenate([[r for r in fixed if r < T], rng.integers(0, T, n)]))


def test_prefill_kimi_k2_bf16_full_size_sampled():
    cfg = config(1)
    _check_prefill(cfg, synth.seed_of(1), rows=_sample_rows(cfg["T"], np.random.default_rng(1)))


def _check_entries_every_row_tile(cfg, inp, run):
    """Cache entries [c | k_pe] of one row in every 256-row tile of the B*T rows: at
    the full sizes the k_pe columns of the joint down-projection are a separate
    split-K product."""
    d = oracle_dims(cfg)
    e4m3 = cfg["weight"] == "e4m3"
    fp8 = {"wkv_a": quant_weight_block128(inp["w"]["wkv_a"])} if e4m3 else None
    T, ntile = cfg["T"], cfg["B"] * cfg["T"] // 256
    rows = [256 * k + (37 * k) % 256 for k in range(ntile)]
    cache = run.kv_cache.float().cpu().numpy()
    for b in range(cfg["B"]):
        ts = np.array([m - b * T for m in rows if b * T <= m < (b + 1) * T])
        entry = mla.latent_path(inp["x"][b][ts], inp["w"], d, ts, fp8=fp8)
        if e4m3:   # fp8 bar: a latent whose fp32 and fp64 values round apart can land on a neighbouring code
            assert_parity(cache[b][ts], e4m3_entries(entry, cfg["kv_lora_rank"]), tol=FP8_TOL, cos=0.999,
                          what=f"kv_cache_out rows of sequence {b}")
        else:
            assert_parity(cache[b][ts], entry, what=f"kv_cache_out rows of sequence {b}")


def test_prefill_kimi_k2_fp8_full_size_sampled():
    cfg = config(2)
    inp, run = _check_prefill(cfg, synth.seed_of(2), rows=_sample_rows(cfg["T"], np.random.default_rng(2), 4),
                              batches=[0, 3], tol=FP8_TOL, cos=0.999)
    _check_entries_every_row_tile(cfg, inp, run)


def test_prefill_dsv32_sparse_full_size_sampled():
    cfg = config(3)
    inp, run = _check_prefill(cfg, synth.seed_of(3), rows=_sample_rows(cfg["T"], np.random.default_rng(3)))
    _check_entries_every_row_tile(cfg, inp, run)


def _check_decode(cfg, seed, cache_len=None, seqs=None, max_len=None):
    fp8 = cfg.get("weight") == "e4m3"
    tol, cos = (FP8_TOL, 0.999) if fp8 else (BF16_TOL, 0.9999)
    inp = synth.gen_decode(cfg, seed, max_len=max_len)
    if cache_len is not None:
        inp["cache_len"] = np.asarray(cache_len, dtype=np.int32)
    run = runner.Decode(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    if fp8 and cfg["B"] * cfg["cache_len"] <= 4096:
        # e4m3: the unabsorbed definition (every Linear as prefill applies it, kv_b on each cached latent)
        ref, entry = mla.mla_decode(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], seqs=seqs, fp8=True,
                                    topk_idx=inp.get("topk_idx"))
    else:
        # its exact reassociation (pinned equal to it on the CPU), much cheaper at full size
        ref, entry = mla.mla_decode_absorbed(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], seqs=seqs,
                                             fp8=fp8, topk_idx=inp.get("topk_idx"))
    got = run.out.float().cpu().numpy()
    sel = np.arange(cfg["B"]) if seqs is None else np.asarray(seqs)
    assert_parity(got[sel], ref, tol=tol, cos=cos, what=cfg["name"])
    if fp8:   # the appended entry holds its latent in the e4m3 view
        entry = e4m3_entries(entry, cfg["kv_lora_rank"])
    # the cache changed exactly at slot cache_len[b]; every other slot is bit-identical
    new = run.cache.float().cpu().numpy()
    old = run.cache0.float().cpu().numpy()
    for i, b in enumerate(sel):
        P = int(inp["cache_len"][b])
        keep = np.ones(new.shape[1], dtype=bool)
        keep[P] = False
        np.testing.assert_array_equal(new[b][keep], old[b][keep])
        assert_parity(new[b, P], entry[i], tol=tol, cos=cos, what="appended cache entry")
    return inp, run


def test_decode_small_varied_lengths():
    cfg = dict(name="dec_small", mode="decode", B=6, cache_len=40, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=64, act="bf16", weight="bf16")
    _check_decode(cfg, 31, cache_len=[0, 1, 31, 32, 33, 40], max_len=48)


def test_decode_dsv32_full_size():
    cfg = config(4)
    _check_decode(cfg, synth.seed_of(4), max_len=1024)


def test_decode_fp8_small_varied_lengths():
    cfg = dict(name="dec_small_fp8", mode="decode", B=6, cache_len=40, dim=1024, q_lora_rank=256,
               kv_lora_rank=512, n_heads=64, act="bf16", weight="e4m3")
    _check_decode(cfg, 33, cache_len=[0, 1, 31, 32, 33, 40], max_len=48)


def test_decode_fp8_dsv32_full_size_sampled():
    # e4m3 weights at the DeepSeek-V3.2-Exp decode shapes (B = 128, 1000 cached)
    cfg = config(4, weight="e4m3")
    _check_decode(cfg, synth.seed_of(4), max_len=1024, seqs=[0, 1, 37, 64, 100, 127])


@pytest.mark.parametrize("weight", ["bf16", "e4m3"])
def test_decode_batch_past_128_rows(weight):
    # 140 sequences: the projections run in two 128-row chunks, the absorb kernel
    # in two sequence blocks and the attention grid ends in a partial group of 8
    cfg = dict(name="dec_b140", mode="decode", B=140, cache_len=20, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=64, act="bf16", weight=weight)
    lens = [(7 * b) % 21 for b in range(140)]
    _check_decode(cfg, 43 if weight == "bf16" else 44, cache_len=lens, max_len=24,
                  seqs=[0, 1, 5, 127, 128, 129, 138, 139])


def test_decode_out_of_range_length_gives_zero_row():
    cfg = dict(name="dec_bad", mode="decode", B=3, cache_len=10, dim=512, q_lora_rank=128, kv_lora_rank=512,
               n_heads=64, act="bf16", weight="bf16")
    inp = synth.gen_decode(cfg, 32, max_len=16)
    inp["cache_len"] = np.array([5, 16, -1], dtype=np.int32)
    run = runner.Decode(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    out = run.out.float().cpu().numpy()
    assert (out[1] == 0).all() and (out[2] == 0).all()
    assert torch.equal(run.cache[1:], run.cache0[1:])
    d = oracle_dims(cfg)
    ref, _ = mla.mla_decode_absorbed(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], seqs=[0])
    assert_parity(out[:1], ref)


def test_prefill_is_deterministic():
    cfg = small_cfg(T=257, topk=32)
    inp = synth.gen_prefill(cfg, 41)
    run = runner.Prefill(cfg, inp)
    run.run()
    a = run.out.clone()
    run.run()
    torch.cuda.synchronize()
    assert torch.equal(a, run.out)


# --------------------------------------------------------------------------
# prefill over a non-empty cache (chunked prefill)

def _check_chunk(cfg, seed, start_pos, max_len, rows=None, tol=BF16_TOL, cos=0.9999):
    inp = synth.gen_chunk(cfg, seed, start_pos, max_len)
    run = runner.PrefillCached(cfg, inp, start_pos)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    ref, entries = mla.mla_prefill_cached(inp["x"], inp["w"], d, inp["cache"][:, :start_pos], start_pos,
                                          topk_idx=inp["topk_idx"], rows=rows, fp8=cfg["weight"] == "e4m3")
    got = run.out.float().cpu().numpy()
    assert_parity(got if rows is None else got[:, rows], ref, tol=tol, cos=cos, what=f"{cfg['name']} chunk")
    cache = run.cache.float().cpu().numpy()
    T = cfg["T"]
    if cfg["weight"] == "e4m3":   # the chunk's entries hold their latents in the e4m3 view
        entries = e4m3_entries(entries, cfg["kv_lora_rank"])
    assert_parity(cache[:, start_pos:start_pos + T], entries, tol=tol, cos=cos, what="chunk cache entries")
    # rows before the chunk are read only, rows after it untouched
    np.testing.assert_array_equal(cache[:, :start_pos], inp["cache"][:, :start_pos])
    assert not cache[:, start_pos + T:].any()
    return run


def test_prefill_cached_small_bf16():
    _check_chunk(small_cfg(T=100, B=2), 41, start_pos=150, max_len=300)


def test_prefill_cached_small_topk_ragged():
    _check_chunk(small_cfg(T=90, B=1, topk=40, n_heads=2), 42, start_pos=77, max_len=200)


def test_prefill_cached_small_fp8():
    _check_chunk(small_cfg(T=70, B=2, dim=1024, q_lora_rank=512, kv_lora_rank=512, n_heads=2, weight="e4m3"), 43,
                 start_pos=64, max_len=160, tol=FP8_TOL, cos=0.999)


def test_prefill_cached_start_zero_and_single_token():
    _check_chunk(small_cfg(T=65, B=2), 44, start_pos=0, max_len=100)
    _check_chunk(small_cfg(T=1, B=3), 45, start_pos=33, max_len=40)


def test_prefill_chunks_chain_to_one_prefill():
    """Two chunks through one device cache give the rows of one prefill over both."""
    cfg = small_cfg(T=200, B=2)
    inp = synth.gen_prefill(cfg, 46)
    d = oracle_dims(cfg)
    ref = mla.mla_prefill(inp["x"], inp["w"], d)
    P = 120
    parts = []
    cache = None
    for lo, hi in ((0, P), (P, 200)):
        c = dict(cfg, T=hi - lo)
        sub = dict(x=inp["x"][:, lo:hi], w=inp["w"], topk_idx=None,
                   cache=np.zeros((2, 256, cfg["kv_lora_rank"] + 64), dtype=np.float32))
        run = runner.PrefillCached(c, sub, lo)
        if cache is not None:
            run.cache.copy_(cache)
        run.run()
        torch.cuda.synchronize()
        cache = run.cache
        parts.append(run.out.float().cpu().numpy())
    assert_parity(np.concatenate(parts, axis=1), ref, what="chained chunks")


def test_prefill_cached_kimi_k2_full_size_sampled():
    # a 2048-token chunk after 2048 cached tokens, Kimi-K2 shapes
    cfg = config(1)
    rows = _sample_rows(cfg["T"], np.random.default_rng(5))
    _check_chunk(cfg, 47, start_pos=2048, max_len=4096, rows=rows)


def test_prefill_cached_rejects_overflowing_chunk():
    from head_latent_attention_fwd_amd import api
    cfg = small_cfg(T=10, B=1)
    inp = synth.gen_chunk(cfg, 48, 5, max_len=16)
    run = runner.PrefillCached(cfg, inp, 5)
    run.start_pos = 7        # 7 + 10 > 16
    with pytest.raises(api.MlaError):
        run.run()


# --------------------------------------------------------------------------
# selected keys: decode over a selection, prefill in the absorbed latent form

def test_decode_sparse_small_varied_lengths():
    cfg = dict(name="dec_sparse", mode="decode", B=6, cache_len=40, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=64, act="bf16", weight="bf16", topk=9)
    inp_len = [0, 1, 31, 32, 33, 40]
    inp = synth.gen_decode(cfg, 71, max_len=48)
    inp["cache_len"] = np.asarray(inp_len, dtype=np.int32)
    rng = np.random.default_rng(72)
    # rows mix valid picks, -1 padding and positions past the row's own slot (ignored)
    idx = np.full((6, 9), -1, dtype=np.int32)
    for b, P in enumerate(inp_len):
        k = min(P + 1, 7)
        idx[b, :k] = rng.choice(P + 1, k, replace=False)
        idx[b, 8] = min(P + 3, 47)
    inp["topk_idx"] = idx
    run = runner.Decode(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    ref, _ = mla.mla_decode_absorbed(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], topk_idx=idx)
    assert_parity(run.out.float().cpu().numpy(), ref, what="sparse decode")


def test_decode_sparse_cache_past_2048():
    # 3000 cached positions, 2048 selected per sequence
    cfg = dict(name="dec_sparse_long", mode="decode", B=4, cache_len=3000, dim=1024, q_lora_rank=256,
               kv_lora_rank=512, n_heads=128, act="bf16", weight="bf16", topk=2048)
    _check_decode(cfg, 73, max_len=3008)


def test_decode_sparse_dsv32_full_size_sampled():
    cfg = config(4, cache_len=4000, topk=2048)
    _check_decode(cfg, synth.seed_of(4), max_len=4096, seqs=[0, 1, 63, 127])


def _check_absorbed(cfg, seed, rows=None):
    inp = synth.gen_prefill(cfg, seed)
    run = runner.PrefillAbsorbed(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    ref = mla.mla_prefill(inp["x"], inp["w"], d, topk_idx=inp["topk_idx"], rows=rows)
    got = run.out.float().cpu().numpy()
    assert_parity(got if rows is None else got[:, rows], ref, what=f"{cfg['name']} absorbed")
    return inp, run


def test_prefill_absorbed_small_topk():
    inp, run = _check_absorbed(small_cfg(T=300, B=2, topk=40, n_heads=64), 74)
    d = oracle_dims(small_cfg())
    entry = mla.latent_path(inp["x"][1], inp["w"], d, np.arange(300))
    assert_parity(run.kv_cache[1].float().cpu().numpy(), entry, what="kv_cache_out")


def test_prefill_absorbed_selection_wider_than_rows():
    # topk above T: every row keeps its whole causal prefix
    _check_absorbed(small_cfg(T=100, B=1, topk=128, n_heads=128), 75)


def test_prefill_absorbed_dsv32_full_size_sampled():
    cfg = config(3)
    _check_absorbed(cfg, synth.seed_of(3), rows=_sample_rows(cfg["T"], np.random.default_rng(3)))


def test_prefill_cached_topk_fp8_batched():
    # a selection over absolute positions, e4m3 weights, two sequences
    _check_chunk(small_cfg(T=96, B=2, dim=1024, q_lora_rank=512, kv_lora_rank=512, n_heads=2, weight="e4m3",
                           topk=24), 49, start_pos=130, max_len=256, tol=FP8_TOL, cos=0.999)


def test_decode_sparse_fp8_dsv32_sampled():
    # e4m3 weights, 3000 cached, top-2048 per sequence, DeepSeek-V3.2-Exp shapes
    cfg = config(4, weight="e4m3", cache_len=3000, topk=2048)
    _check_decode(cfg, 76, max_len=3008, seqs=[0, 50, 127])


def test_prefill_absorbed_batched_ragged():
    # two sequences, T not a multiple of any tile, selection narrower than most rows
    _check_absorbed(small_cfg(B=2, T=77, topk=9, n_heads=64), 77)


def test_decode_graph_replay_matches_eager():
    """The decode step captured in a HIP graph and replayed (with eager work in
    between) gives the eager result every time."""
    cfg = dict(name="dec_graph", mode="decode", B=8, cache_len=100, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=64, act="bf16", weight="bf16")
    inp = synth.gen_decode(cfg, 78, max_len=128)
    run = runner.Decode(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    eager = run.out.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        run.run(stream=stream)          # warm-up on the capture stream
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            run.run(stream=stream)
    for i in range(3):
        run.out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out, eager), f"replay {i}"
        run.run()                        # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(run.out, eager)


def test_one_token_chunk_matches_decode_on_the_gpu():
    """A one-token chunk after P cached tokens and the decode step for the same
    token go through different kernels (dense prefill attention vs the latent
    decode attention) and must agree with each other and the oracle."""
    cfg = dict(name="chunk1", mode="prefill", B=3, T=1, dim=1024, q_lora_rank=256, kv_lora_rank=512, n_heads=64,
               act="bf16", weight="bf16", topk=0, cache_len=150)
    P, max_len = 150, 160
    inp = synth.gen_chunk(cfg, 79, P, max_len)
    chunk = runner.PrefillCached(cfg, inp, P)
    chunk.run()
    dec_inp = dict(x=inp["x"][:, 0], w=inp["w"], cache=inp["cache"], cache_len=np.full(3, P, dtype=np.int32))
    dec = runner.Decode(dict(cfg, mode="decode"), dec_inp)
    dec.run()
    torch.cuda.synchronize()
    a = chunk.out[:, 0].float().cpu().numpy()
    b = dec.out.float().cpu().numpy()
    d = oracle_dims(cfg)
    ref, _ = mla.mla_decode(inp["x"][:, 0], inp["w"], d, inp["cache"], np.full(3, P))
    assert_parity(a, ref, what="one-token chunk")
    assert_parity(b, ref, what="decode")
    assert_parity(a, b, what="chunk vs decode")
    # both wrote the same cache entry at slot P
    assert_parity(chunk.cache[:, P].float().cpu().numpy(), dec.cache[:, P].float().cpu().numpy(), what="entry")


def test_prefill_graph_replay_matches_eager():
    """The whole prefill (top-k, bf16) captured in a HIP graph and replayed with
    eager work in between reproduces the eager output exactly."""
    cfg = small_cfg(T=150, B=2, topk=20, n_heads=4)
    inp = synth.gen_prefill(cfg, 80)
    run = runner.Prefill(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    eager, eager_cache = run.out.clone(), run.kv_cache.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        run.run(stream=stream)
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            run.run(stream=stream)
    for i in range(3):
        run.out.zero_()
        run.kv_cache.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.out, eager) and torch.equal(run.kv_cache, eager_cache), f"replay {i}"
        run.run()
        torch.cuda.synchronize()


def test_decode_sparse_repeated_and_unsorted_positions():
    """A selection is a set: repeated positions count once and the order of the
    list does not matter (DeepSeek-V3.2-Exp · Sparse attention, Code: picks are
    scattered as 0 into a -inf mask)."""
    cfg = dict(name="dec_dup", mode="decode", B=4, cache_len=300, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=128, act="bf16", weight="bf16", topk=64)
    inp = synth.gen_decode(cfg, 81, max_len=320)
    inp["cache_len"] = np.array([300, 5, 299, 150], dtype=np.int32)
    rng = np.random.default_rng(82)
    idx = np.full((4, 64), -1, dtype=np.int32)
    for b, P in enumerate(inp["cache_len"]):
        pick = rng.choice(P + 1, min(P + 1, 30), replace=False)
        lst = np.concatenate([pick, pick[:10], pick[:3], [P + 7, -1]])   # repeats, a future slot, padding
        rng.shuffle(lst)
        idx[b, :len(lst)] = lst
    inp["topk_idx"] = idx
    run = runner.Decode(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    ref, _ = mla.mla_decode(inp["x"], inp["w"], d, inp["cache"], inp["cache_len"], topk_idx=idx)
    assert_parity(run.out.float().cpu().numpy(), ref, what="decode, repeated selection")
    # the same selection without repeats gives the same output bit for bit
    uniq = np.full_like(idx, -1)
    for b in range(4):
        u = np.unique(idx[b][idx[b] >= 0])
        uniq[b, :len(u)] = u
    run.topk.copy_(torch.from_numpy(uniq))
    first = run.out.clone()
    run.cache.copy_(run.cache0)
    run.run()
    torch.cuda.synchronize()
    assert torch.equal(run.out, first)


def test_prefill_absorbed_repeated_positions():
    cfg = small_cfg(B=1, T=120, topk=24, n_heads=64)
    inp = synth.gen_prefill(cfg, 83)
    idx = inp["topk_idx"].copy()
    rng = np.random.default_rng(84)
    for s in range(120):   # overwrite the padding and a few picks with repeats, then shuffle the row
        row = idx[0, s]
        live = row[row >= 0]
        if len(live) > 2:
            row[-3:] = live[:3]
        rng.shuffle(row)
    inp["topk_idx"] = idx
    run = runner.PrefillAbsorbed(cfg, inp)
    run.run()
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    ref = mla.mla_prefill(inp["x"], inp["w"], d, topk_idx=idx)
    assert_parity(run.out.float().cpu().numpy(), ref, what="absorbed prefill, repeated selection")


def test_e4m3_prefill_cache_feeds_decode():
    """With e4m3 weights the prefill writes each latent in its e4m3 view and the
    decode reads the cache as it is: a decode step over the cache a prefill left
    behind equals the oracle's e4m3 decode over the oracle's own plain cache
    entries of the same tokens."""
    cfg = small_cfg(B=2, T=40, dim=1024, q_lora_rank=256, kv_lora_rank=512, n_heads=64, weight="e4m3")
    inp = synth.gen_prefill(cfg, 91)
    pre = runner.Prefill(cfg, inp)
    pre.run()
    B, T, max_len = cfg["B"], cfg["T"], 48
    cache = torch.zeros((B, max_len, 576), dtype=torch.bfloat16, device="cuda")
    cache[:, :T] = pre.kv_cache
    x_new = synth.round_bf16(np.random.default_rng(92).standard_normal((B, cfg["dim"])))
    cos, sin = api.mla_rope_table(max_len)
    out = torch.empty((B, cfg["dim"]), dtype=torch.bfloat16, device="cuda")
    ws = api.workspace(api.mla_decode_workspace_size(pre.dims, pre.wdt, B, max_len), "cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    api.mla_decode(pre.dims, pre.weights, runner.to_dev(x_new, torch.bfloat16), cache, lens, cos, sin, out, ws)
    torch.cuda.synchronize()
    d = oracle_dims(cfg)
    fp8 = {"wkv_a": quant_weight_block128(inp["w"]["wkv_a"])}
    ref_cache = np.zeros((B, max_len, 576))
    for b in range(B):
        ref_cache[b, :T] = mla.latent_path(inp["x"][b], inp["w"], d, np.arange(T), fp8=fp8)
    ref, _ = mla.mla_decode(x_new, inp["w"], d, ref_cache, np.full(B, T), fp8=True)
    assert_parity(out.float().cpu().numpy(), ref, tol=FP8_TOL, cos=0.999, what="decode over an e4m3 prefill's cache")


@pytest.mark.parametrize("weight,T,dim,q_lora", [("e4m3", 13300, 1024, 512), ("bf16", 8092, 7168, 1536)])
def test_prefill_kpe_split_ragged_rows(weight, T, dim, q_lora):
    """Row counts that are not a multiple of the 256-row tile, at sizes where the
    k_pe columns of the joint down-projection run as their own split-K product
    (the launch schedule decides it from the shapes): sampled rows and one
    cache entry per row tile against the oracle."""
    cfg = small_cfg(B=1, T=T, dim=dim, q_lora_rank=q_lora, kv_lora_rank=512, n_heads=2, weight=weight)
    tol, cos = (FP8_TOL, 0.999) if weight == "e4m3" else (BF16_TOL, 0.9999)
    inp, run = _check_prefill(cfg, 93, rows=_sample_rows(T, np.random.default_rng(93), 6), tol=tol, cos=cos)
    _check_entries_every_row_tile(cfg, inp, run)
