"""Per-kernel parity of the HIP library against the fp64 oracle (GPU)."""
import numpy as np
import pytest
import torch

from head_latent_attention_fwd_amd import api, synth
from oracle import fp8, mask, mla

from helpers import BF16_TOL, F32_TOL, FP8_TOL, assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)


def test_rope_table_matches_definition():
    c, s = api.mla_rope_table(9000)
    th = mla.rope_angles(np.arange(9000))
    np.testing.assert_allclose(c.cpu().numpy(), np.cos(th), atol=2e-7, rtol=0)
    np.testing.assert_allclose(s.cpu().numpy(), np.sin(th), atol=2e-7, rtol=0)


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (130, 300, 200), (257, 2112, 7168), (2048, 7168, 2048),
                                   (64, 24576, 1536)])
@pytest.mark.parametrize("cdt", [torch.bfloat16, torch.float32])
def test_gemm_bf16(M, N, K, cdt):
    rng = np.random.default_rng(M * 7 + N + K)
    a = synth.round_bf16(rng.standard_normal((M, K)))
    w = synth.round_bf16(rng.standard_normal((N, K)) / np.sqrt(K))
    C = torch.empty((M, N), dtype=cdt, device=DEV)
    api.gemm_bf16(dev(a, torch.bfloat16), dev(w, torch.bfloat16), C)
    assert_parity(C.float().cpu().numpy(), mla.linear(a, w), what=f"gemm {M}x{N}x{K}")


def test_gemm_bf16_strided_operands():
    rng = np.random.default_rng(1)
    a = synth.round_bf16(rng.standard_normal((70, 600)))
    w = synth.round_bf16(rng.standard_normal((90, 600)))
    A = dev(a, torch.bfloat16)[:, 64:576]            # row stride 600, K = 512
    W = dev(w, torch.bfloat16)[:, 64:576]
    C = torch.zeros((70, 100), dtype=torch.float32, device=DEV)[:, :90]
    api.gemm_bf16(A, W, C)
    assert_parity(C.cpu().numpy(), mla.linear(a[:, 64:576], w[:, 64:576]))


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (130, 256, 512), (64, 384, 128)])
def test_gemm_f32(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    api.gemm_f32(dev(a, torch.float32), dev(w, torch.float32), C)
    assert_parity(C.cpu().numpy(), mla.linear(a, w), tol=F32_TOL, cos=0.999999)


def _act_with_edges(M, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)) * np.exp(rng.uniform(-8, 8, (M, 1)))
    a[0, :128] = 0.0                                  # all-zero group
    a[1, 5] = 1e30 if K > 5 else a[1, 0]              # one huge element
    a[2, 128:256] = 1e-30 if K >= 256 else 0.0        # subnormal-sized group
    return synth.round_bf16(a)


@pytest.mark.parametrize("M,K", [(300, 7168), (17, 128), (64, 8192)])
def test_quant_1x128_bit_exact(M, K):
    a = _act_with_edges(M, K, M + K)
    q, s = api.mla_quant_e4m3_1x128(dev(a, torch.bfloat16))
    rq, rs = fp8.quant_act_1x128(a, quotient="f32")
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_latent_e4m3_view():
    """Each 128-group of a cache row's latent replaced by its 1x128 e4m3 value
    (kv_b's quantised input); the rotary part untouched. The view quantises back
    to the codes of the plain latent (a fixed point of the quantiser) and sits
    within one bf16 step of code x scale."""
    B, S, L = 3, 40, 512
    lat = _act_with_edges(B * S, L, 7).reshape(B, S, L)
    rope = synth.round_bf16(np.random.default_rng(8).standard_normal((B, S, 64)))
    cache = dev(np.concatenate([lat, rope], axis=-1), torch.bfloat16)
    api.mla_latent_e4m3_view(cache, L)
    got = cache.float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got[..., L:], rope)
    ref = fp8.quant_dequant_act(lat.reshape(-1, L)).reshape(B, S, L)
    assert (np.abs(got[..., :L] - ref) <= 2.0 ** -7 * np.abs(ref)).all()
    q_view, s_view = fp8.quant_act_1x128(got[..., :L].reshape(-1, L), quotient="f32")
    q_lat, s_lat = fp8.quant_act_1x128(lat.reshape(-1, L), quotient="f32")
    np.testing.assert_array_equal(s_view, s_lat)
    np.testing.assert_array_equal(q_view, q_lat)


@pytest.mark.parametrize("N,K", [(576, 7168), (130, 200), (1536, 7168)])
def test_quant_block128_bit_exact(N, K):
    rng = np.random.default_rng(N * K)
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    w[:128, :128] = 0.0
    q, s = api.mla_quant_e4m3_block128(dev(w, torch.float32))
    rq, rs = fp8.quant_weight_block128(w)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("M,N,K", [(130, 576, 7168), (256, 1024, 1536), (33, 200, 512)])
def test_gemm_fp8_blockscaled(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = synth.round_bf16(rng.standard_normal((M, K)))
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    Aq, As = api.mla_quant_e4m3_1x128(dev(a, torch.bfloat16))
    Wq, Ws = api.mla_quant_e4m3_block128(dev(w, torch.float32))
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    api.gemm_fp8_blockscaled(Aq, As, Wq, Ws, C)
    ac, as_ = fp8.quant_act_1x128(a, quotient="f32")
    wc, ws = fp8.quant_weight_block128(w)
    ref = fp8.fp8_gemm(ac, as_, wc, ws)
    # identical codes; fp32 accumulation inside the fp8 MFMA and the promotion
    # differ from fp64 by ~2e-5 of max|C| (measured)
    assert_parity(C.cpu().numpy(), ref, tol=1e-4, cos=0.999999, what="fp8 gemm")


@pytest.mark.parametrize("M,N,K,out", [(4352, 4096, 512, torch.bfloat16), (600, 2112, 1024, torch.float32),
                                       (1000, 1280, 2048, torch.bfloat16)])
def test_gemm_fp8_blockscaled_many_tiles(M, N, K, out):
    # more 256 x 256 tiles than CUs (a second round, whose first K groups the
    # first round's tiles fetch into L2 ahead of it), a ragged last row tile, a
    # 64-wide last column tile (N = 2112), bf16 and fp32 outputs; all three
    # take the short-K loop (at most 16 groups)
    rng = np.random.default_rng(M * 7 + N + K)
    a = synth.round_bf16(rng.standard_normal((M, K)))
    w = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    Aq, As = api.mla_quant_e4m3_1x128(dev(a, torch.bfloat16))
    Wq, Ws = api.mla_quant_e4m3_block128(dev(w, torch.float32))
    C = torch.full((M, N), 7.0, dtype=out, device=DEV)
    api.gemm_fp8_blockscaled(Aq, As, Wq, Ws, C)
    ac, as_ = fp8.quant_act_1x128(a, quotient="f32")
    wc, ws = fp8.quant_weight_block128(w)
    ref = fp8.fp8_gemm(ac, as_, wc, ws)
    if out == torch.bfloat16:
        ref = synth.round_bf16(ref)
    assert_parity(C.float().cpu().numpy(), ref, tol=1e-4 if out == torch.float32 else 8e-3, cos=0.999999,
                  what="fp8 gemm, many tiles")


def test_rmsnorm_rope_kv_and_q_layouts():
    rng = np.random.default_rng(3)
    T = 77
    kv = synth.round_bf16(rng.standard_normal((T, 576)) * 3)
    gamma = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    c, s = api.mla_rope_table(128)
    out = torch.empty((T, 576), dtype=torch.bfloat16, device=DEV)
    api.rmsnorm_rope(dev(kv, torch.bfloat16), out, norm_dim=512, gamma=dev(gamma, torch.float32), eps=1e-6,
                     rope_off=512, rope_heads=1, rope_stride=64, rope_cos=c, rope_sin=s, pos_period=T)
    ref = mla.rmsnorm_rope_rows(kv, 512, gamma, 1e-6, 512, 1, 64, np.arange(T), 10000.0)
    assert_parity(out.float().cpu().numpy(), ref, what="kv norm+rope")
    # q layout: rope on 5 heads of 192, at offset 128, positions from a device array
    q = synth.round_bf16(rng.standard_normal((T, 5 * 192)))
    pos = rng.integers(0, 128, T).astype(np.int32)
    qd = dev(q, torch.bfloat16)
    api.rmsnorm_rope(qd, qd, rope_off=128, rope_heads=5, rope_stride=192, rope_cos=c, rope_sin=s,
                     pos=dev(pos, torch.int32))
    ref = mla.rmsnorm_rope_rows(q, 0, None, 0, 128, 5, 192, pos, 10000.0)
    assert_parity(qd.float().cpu().numpy(), ref, what="q rope in place")
    # untouched elements stay bit-identical
    got = qd.float().cpu().numpy().reshape(T, 5, 192)[:, :, :128]
    np.testing.assert_array_equal(got, q.reshape(T, 5, 192)[:, :, :128])


def test_rmsnorm_f32():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 1536)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(1536)).astype(np.float32)
    out = torch.empty((9, 1536), dtype=torch.float32, device=DEV)
    api.rmsnorm_rope(dev(x, torch.float32), out, norm_dim=1536, gamma=dev(g, torch.float32), eps=1e-6)
    assert_parity(out.cpu().numpy(), mla.rmsnorm(x, g, 1e-6), tol=1e-6, cos=0.9999999)


@pytest.mark.parametrize("B,T,k", [(2, 100, 9), (1, 4100, 2048)])
def test_topk_bitmask_bit_exact(B, T, k):
    rng = np.random.default_rng(T)
    idx = rng.integers(-3, T + 5, size=(B, T, k)).astype(np.int32)
    idx[:, :, 0] = np.arange(T)[None, :]
    m = api.mla_topk_to_bitmask(dev(idx, torch.int32))
    ref = mask.topk_bitmask(idx, T)
    np.testing.assert_array_equal(m.cpu().numpy().view(np.uint32), ref)


def test_boundary_errors_do_not_launch():
    d = api.make_dims(512, 128, 64, 2)
    d.qk_nope_head_dim = 96
    assert api.mla_prefill_workspace_size(d, 0, 0, 1, 1) == 0
    a = torch.zeros((4, 100), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(api.MlaError) as e:
        api.mla_quant_e4m3_1x128(a, scales=torch.zeros((4, 1), dtype=torch.float32, device=DEV))
    assert e.value.code == api.MLA_UNSUPPORTED


@pytest.mark.parametrize("B,T,H,k", [(2, 190, 3, 0), (1, 300, 2, 37), (1, 4096, 1, 2048), (3, 5, 2, 0)])
def test_prefill_attention_step(B, T, H, k):
    rng = np.random.default_rng(B * T + H + k)
    Tp = api.pad64(T)
    q = synth.round_bf16(rng.standard_normal((B * T, H * 192)))
    kn = synth.round_bf16(rng.standard_normal((B, H, T, 128)))
    v = synth.round_bf16(rng.standard_normal((B, H, T, 128)))
    kp = synth.round_bf16(rng.standard_normal((B, T, 64)))
    idx = synth.draw_topk(rng, B, T, k) if k else None
    m = api.mla_topk_to_bitmask(dev(idx, torch.int32)) if k else None
    # device layouts, with junk (NaN) in the padding keys: the call must zero it
    KN = torch.full((B, H, Tp, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    KN[:, :, :T] = dev(kn, torch.bfloat16)
    VT = torch.full((B, H, 128, Tp), float("nan"), dtype=torch.bfloat16, device=DEV)
    VT[:, :, :, :T] = dev(np.ascontiguousarray(v.transpose(0, 1, 3, 2)), torch.bfloat16)
    KP = torch.full((B, Tp, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    KP[:, :T] = dev(kp, torch.bfloat16)
    out = torch.empty((B * T, H * 128), dtype=torch.bfloat16, device=DEV)
    api.mla_prefill_attention(dev(q, torch.bfloat16), KN, VT, KP, out, B, T, H, mask=m)
    got = out.float().cpu().numpy().reshape(B, T, H, 128)
    rows = sorted(set([0, T // 3, T - 1] + [int(r) for r in rng.integers(0, T, 6)]))
    sc = 192.0 ** -0.5
    for b in range(B):
        qq = q.reshape(B, T, H, 192)[b]
        ref = np.stack([mla.attend_row(qq[s, :, :128], qq[s, :, 128:], kn[b].transpose(1, 0, 2), kp[b],
                                       v[b].transpose(1, 0, 2),
                                       mla.live_keys(s, None if idx is None else idx[b, s]), sc)[0] for s in rows])
        assert_parity(got[b, rows], ref, what=f"attention b={b}")


def test_decode_attention_step():
    rng = np.random.default_rng(9)
    B, H, max_len = 5, 128, 300
    lens = np.array([0, 31, 32, 299, 150], dtype=np.int32)
    ql = synth.round_bf16(rng.standard_normal((B, H, 576)) * 0.3)
    cache = synth.round_bf16(rng.standard_normal((B, max_len, 576)))
    ol = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    api.mla_decode_attention(dev(ql, torch.bfloat16), dev(cache, torch.bfloat16), dev(lens, torch.int32), ol)
    got = ol.float().cpu().numpy()
    for b in range(B):
        C = cache[b, :lens[b] + 1].astype(np.float64)
        z = ql[b].astype(np.float64) @ C.T * 192.0 ** -0.5
        ref = mla.softmax_over_live(z) @ C[:, :512]
        assert_parity(got[b], ref, what=f"decode attention b={b}")


@pytest.mark.parametrize("B,H,max_len,lens", [(1, 128, 4100, [4099]), (2, 64, 1100, [1000, 17]),
                                               (300, 128, 40, None)])
def test_decode_attention_key_runs(B, H, max_len, lens):
    """Key ranges cut into several runs (one long sequence: 16 runs; two
    sequences of different lengths; many sequences: one run), merged in order."""
    rng = np.random.default_rng(B + H + max_len)
    lens = np.asarray(lens if lens is not None else rng.integers(0, max_len, B), dtype=np.int32)
    ql = synth.round_bf16(rng.standard_normal((B, H, 576)) * 0.3)
    cache = synth.round_bf16(rng.standard_normal((B, max_len, 576)))
    ol = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    api.mla_decode_attention(dev(ql, torch.bfloat16), dev(cache, torch.bfloat16), dev(lens, torch.int32), ol)
    got = ol.float().cpu().numpy()
    for b in sorted(set([0, B - 1, B // 2])):
        C = cache[b, :lens[b] + 1].astype(np.float64)
        z = ql[b].astype(np.float64) @ C.T * 192.0 ** -0.5
        ref = mla.softmax_over_live(z) @ C[:, :512]
        assert_parity(got[b], ref, what=f"decode attention runs b={b}")


def _prefill_attention_every_tile(B, T, H, k, seed):
    """mla_prefill_attention at a full workload shape, one query row from every
    128-row tile of every head (all heads of a row are compared), against the
    oracle's attend_row (DeepSeek-V3.2-Exp · Sparse attention, Code)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    Tp = api.pad64(T)
    bf = torch.bfloat16
    Q = torch.randn((B * T, H * 192), generator=g, device=DEV).to(bf)
    KN = torch.randn((B, H, Tp, 128), generator=g, device=DEV).to(bf)
    VT = torch.randn((B, H, 128, Tp), generator=g, device=DEV).to(bf)
    KP = torch.randn((B, Tp, 64), generator=g, device=DEV).to(bf)
    rng = np.random.default_rng(seed)
    idx = synth.draw_topk(rng, B, T, k) if k else None
    m = api.mla_topk_to_bitmask(dev(idx, torch.int32)) if k else None
    out = torch.empty((B * T, H * 128), dtype=bf, device=DEV)
    api.mla_prefill_attention(Q, KN, VT, KP, out, B, T, H, mask=m)
    torch.cuda.synchronize()
    rows = np.array([min(T - 1, 128 * i + int(rng.integers(0, 128))) for i in range((T + 127) // 128)])
    rows[0], rows[-1] = 0, T - 1
    got = out.view(B, T, H, 128)[:, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    sc = 192.0 ** -0.5
    for b in range(B):
        q = Q.view(B, T, H, 192)[b, torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
        kn = KN[b, :, :T].double().cpu().numpy().transpose(1, 0, 2)      # [T, H, 128]
        v = VT[b, :, :, :T].double().cpu().numpy().transpose(2, 0, 1)    # [T, H, 128]
        kp = KP[b, :T].double().cpu().numpy()
        for i, s in enumerate(rows):
            live = mla.live_keys(int(s), None if idx is None else idx[b, s])
            ref, _ = mla.attend_row(q[i, :, :128], q[i, :, 128:], kn, kp, v, live, sc)
            assert_parity(got[b, i], ref, what=f"attention row {s} (tile {s // 128})")


@pytest.mark.parametrize("k", [0, 24])
def test_prefill_attention_large_logit_jump(k):
    """Later keys outscore a query's first live keys by far more than the fixed
    running max allows (sums beyond 2^64), which sends the workgroup through its
    exact two-pass redo."""
    rng = np.random.default_rng(11 + k)
    B, T, H = 1, 300, 2
    Tp = api.pad64(T)
    q = synth.round_bf16(rng.standard_normal((B * T, H * 192)))
    kn = rng.standard_normal((B, H, T, 128))
    kn[:, :, 100:] *= 40.0
    kn = synth.round_bf16(kn)
    v = synth.round_bf16(rng.standard_normal((B, H, T, 128)))
    kp = synth.round_bf16(rng.standard_normal((B, T, 64)))
    idx = synth.draw_topk(rng, B, T, k) if k else None
    m = api.mla_topk_to_bitmask(dev(idx, torch.int32)) if k else None
    KN = torch.zeros((B, H, Tp, 128), dtype=torch.bfloat16, device=DEV)
    KN[:, :, :T] = dev(kn, torch.bfloat16)
    VT = torch.zeros((B, H, 128, Tp), dtype=torch.bfloat16, device=DEV)
    VT[:, :, :, :T] = dev(np.ascontiguousarray(v.transpose(0, 1, 3, 2)), torch.bfloat16)
    KP = torch.zeros((B, Tp, 64), dtype=torch.bfloat16, device=DEV)
    KP[:, :T] = dev(kp, torch.bfloat16)
    out = torch.empty((B * T, H * 128), dtype=torch.bfloat16, device=DEV)
    api.mla_prefill_attention(dev(q, torch.bfloat16), KN, VT, KP, out, B, T, H, mask=m)
    got = out.float().cpu().numpy().reshape(B, T, H, 128)
    rows = [0, 99, 100, 101, 150, 255, 256, 299]
    qq = q.reshape(B, T, H, 192)[0]
    ref = np.stack([mla.attend_row(qq[s, :, :128], qq[s, :, 128:], kn[0].transpose(1, 0, 2), kp[0],
                                   v[0].transpose(1, 0, 2), mla.live_keys(s, None if idx is None else idx[0, s]),
                                   192.0 ** -0.5)[0] for s in rows])
    assert_parity(got[0, rows], ref, what="attention (logit jump)")


def test_prefill_attention_every_tile_kimi_k2_shape():
    _prefill_attention_every_tile(1, 2048, 64, 0, 91)


def test_prefill_attention_every_tile_dsv32_topk_shape():
    _prefill_attention_every_tile(1, 8192, 128, 2048, 92)


def test_decode_attention_large_logit_jump():
    # later keys outscore the first tile by far more than the fixed-max headroom,
    # which moves the running max and rescales what was accumulated
    rng = np.random.default_rng(10)
    B, H, max_len = 3, 64, 300
    lens = np.array([250, 100, 299], dtype=np.int32)
    ql = synth.round_bf16(rng.standard_normal((B, H, 576)) * 0.3)
    cache = rng.standard_normal((B, max_len, 576))
    cache[0, 64:] *= 40.0
    cache[1, 40:64] *= 40.0
    cache[2, 128:] *= 60.0
    cache = synth.round_bf16(cache)
    ol = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    api.mla_decode_attention(dev(ql, torch.bfloat16), dev(cache, torch.bfloat16), dev(lens, torch.int32), ol)
    got = ol.float().cpu().numpy()
    for b in range(B):
        C = cache[b, :lens[b] + 1].astype(np.float64)
        z = ql[b].astype(np.float64) @ C.T * 192.0 ** -0.5
        ref = mla.softmax_over_live(z) @ C[:, :512]
        assert_parity(got[b], ref, what=f"decode attention (logit jump) b={b}")


@pytest.mark.parametrize("M,hidden,inter", [(33, 192, 320), (300, 1024, 512), (1, 128, 128)])
def test_swiglu_mlp(M, hidden, inter):
    # inter % 128 != 0 takes the two-GEMM path, the rest the paired-tile GEMM
    rng = np.random.default_rng(M + hidden + inter)
    x = synth.round_bf16(rng.standard_normal((M, hidden)))
    wg = synth.round_bf16(rng.standard_normal((inter, hidden)) / np.sqrt(hidden))
    wu = synth.round_bf16(rng.standard_normal((inter, hidden)) / np.sqrt(hidden))
    wd = synth.round_bf16(rng.standard_normal((hidden, inter)) / np.sqrt(inter))
    out = api.mla_swiglu_mlp(dev(x, torch.bfloat16), dev(wg, torch.bfloat16), dev(wu, torch.bfloat16),
                             dev(wd, torch.bfloat16))
    assert_parity(out.float().cpu().numpy(), mla.swiglu_mlp(x, wg, wu, wd), what=f"swiglu {M}x{hidden}x{inter}")


def test_swiglu_mlp_kimi_k2_shared_expert_sampled_rows():
    # full size (2048 tokens, hidden 7168, inter 2048); rows are independent,
    # so the oracle on sampled rows is the oracle of the whole batch there
    M, hidden, inter = 2048, 7168, 2048
    g = torch.Generator(device=DEV).manual_seed(5)
    X = torch.randn((M, hidden), generator=g, device=DEV).to(torch.bfloat16)
    Wg = (torch.randn((inter, hidden), generator=g, device=DEV) / hidden ** 0.5).to(torch.bfloat16)
    Wu = (torch.randn((inter, hidden), generator=g, device=DEV) / hidden ** 0.5).to(torch.bfloat16)
    Wd = (torch.randn((hidden, inter), generator=g, device=DEV) / inter ** 0.5).to(torch.bfloat16)
    out = api.mla_swiglu_mlp(X, Wg, Wu, Wd)
    rows = np.array([0, 1, 255, 256, 1023, 1500, 2046, 2047])
    f64 = lambda t: t.double().cpu().numpy()
    ref = mla.swiglu_mlp(f64(X[rows]), f64(Wg), f64(Wu), f64(Wd))
    assert_parity(out[rows].float().cpu().numpy(), ref, what="swiglu Kimi-K2 shared expert")



@pytest.mark.parametrize("M,hidden,inter", [(300, 1024, 512), (2048, 7168, 2048)])
def test_swiglu_mlp_e4m3(M, hidden, inter):
    # e4m3 weights quantised on the device from fp32 masters; the full Kimi-K2
    # shared-expert size is compared on sampled rows (rows are independent)
    rng = np.random.default_rng(M + 5)
    x = synth.round_bf16(rng.standard_normal((M, hidden)))
    wg = (rng.standard_normal((inter, hidden)) / np.sqrt(hidden)).astype(np.float32)
    wu = (rng.standard_normal((inter, hidden)) / np.sqrt(hidden)).astype(np.float32)
    wd = (rng.standard_normal((hidden, inter)) / np.sqrt(inter)).astype(np.float32)
    q = [api.mla_quant_e4m3_block128(dev(w, torch.float32)) for w in (wg, wu, wd)]
    out = api.mla_swiglu_mlp_e4m3(dev(x, torch.bfloat16), *q)
    rows = np.arange(M) if M <= 512 else np.array([0, 1, 255, 256, 1023, 2047])
    ref = mla.swiglu_mlp(x[rows], wg, wu, wd, fp8=True)
    assert_parity(out.float().cpu().numpy()[rows], ref, tol=FP8_TOL, cos=0.999, what=f"swiglu e4m3 {M}")


@pytest.mark.parametrize("M,N,K", [(128, 7168, 16384), (128, 24576, 1536), (128, 2112, 7168), (5, 200, 640)])
def test_gemm_bf16_decode(M, N, K):
    """Decode-shaped product (the decode step's q_a|kv_a, q_b and wo kernels) against the oracle's Linear."""
    g = torch.Generator(device=DEV).manual_seed(M + N + K)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn((N, K), generator=g, device=DEV) / K ** 0.5).to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    api.gemm_bf16_decode(A, W, C)
    rows = np.unique(np.array([0, M // 2, M - 1]))
    ref = mla.linear(A[rows].double().cpu().numpy(), W.double().cpu().numpy())
    assert_parity(C[rows].float().cpu().numpy(), ref, what=f"decode gemm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(128, 7168, 16384), (128, 24576, 1536), (7, 300, 1024)])
def test_gemm_fp8_decode(M, N, K):
    """Decode-shaped block-scaled e4m3 product against the oracle's block-scaled
    sum over the same codes and scales (Kimi K2 · Down projection, quantization_config)."""
    g = torch.Generator(device=DEV).manual_seed(M * 3 + N + K)
    a = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.randn((N, K), generator=g, device=DEV) / K ** 0.5
    Aq, As = api.mla_quant_e4m3_1x128(a)
    Wq, Ws = api.mla_quant_e4m3_block128(w)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    api.gemm_fp8_decode(Aq, As, Wq, Ws, C)
    rows = np.unique(np.array([0, M // 2, M - 1]))
    ref = fp8.fp8_gemm(Aq[rows].cpu().numpy(), As[rows].cpu().numpy(), Wq.cpu().numpy(), Ws.cpu().numpy())
    assert_parity(C[rows].float().cpu().numpy(), ref, what=f"decode fp8 gemm {M}x{N}x{K}")
