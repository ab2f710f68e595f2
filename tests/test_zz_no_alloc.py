"""The allocation-free decode attention (library-held scratch) against the
workspace entry point it varies, through the C ABI: two calls in a row, the
second with a smaller input."""
import numpy as np
import pytest
import torch

from head_latent_attention_fwd_amd import api, synth

from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _inputs(B, H, max_len, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len, B).astype(np.int32)
    lens[0] = max_len - 1
    ql = synth.round_bf16(rng.standard_normal((B, H, 576)) * 0.3)
    cache = synth.round_bf16(rng.standard_normal((B, max_len, 576)))
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt)
    return dev(ql, torch.bfloat16), dev(cache, torch.bfloat16), dev(lens, torch.int32)


def test_noalloc_matches_the_workspace_entry_point():
    # 127 sequences x 128 heads: two key runs whose partials fill 33.4 MB of the
    # 32 MiB scratch (the largest need the run rule can make); then 2 sequences
    # x 64 heads: 2 runs, a smaller use of the same scratch
    for B, H, max_len, seed in ((127, 128, 1024, 1), (2, 64, 300, 2)):
        ql, cache, lens = _inputs(B, H, max_len, seed)
        need = api.mla_decode_attention_workspace_size(B, H, max_len)
        assert 256 < need <= 32 << 20
        ref = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        api.mla_decode_attention(ql, cache, lens, ref)
        got = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        api.mla_decode_attention_noalloc(ql, cache, lens, got)
        torch.cuda.synchronize()
        assert_parity(got.float().cpu().numpy(), ref.float().cpu().numpy(), what=f"noalloc B={B} H={H}")
        assert torch.equal(got, ref)   # same kernels, same key runs
