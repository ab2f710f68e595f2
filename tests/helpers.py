"""Shared test helpers: the parity bars and small config builders."""
import numpy as np

from head_latent_attention_fwd_amd import synth

# bf16 parity bar: max|gpu - oracle| <= 1e-2 * max|oracle| and cosine >= 0.9999.
BF16_TOL, BF16_COS = 1e-2, 0.9999
# fp8 bar (oracle applies the same block dequantisation): 3e-2 * max|oracle|.
FP8_TOL = 3e-2
# fp32 path: the same arithmetic in fp32 with different summation order; the
# measured error is ~1e-6 of max|oracle|, gated at 1e-4.
F32_TOL = 1e-4


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def cosine(got, ref):
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    return float(g @ r / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300))


def assert_parity(got, ref, tol=BF16_TOL, cos=BF16_COS, what=""):
    e, c = rel_err(got, ref), cosine(got, ref)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{what}: non-finite output"
    assert e <= tol and c >= cos, f"{what}: max rel err {e:.3e} (tol {tol}), cosine {c:.6f} (min {cos})"
    return e, c


def small_cfg(**over):
    cfg = dict(name="small", mode="prefill", B=2, T=200, dim=1024, q_lora_rank=256, kv_lora_rank=512,
               n_heads=3, act="bf16", weight="bf16", topk=0)
    cfg.update(over)
    return cfg


def oracle_dims(cfg):
    from oracle import mla
    return mla.default_dims(cfg["dim"], cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["n_heads"])


def config(i, **over):
    return synth.make_cfg(i, **over)


def e4m3_entries(entries, L):
    """Oracle cache entries in the form the e4m3 calls write them: the latent
    part (first L values) replaced by the value its dynamic 1x128 e4m3
    quantisation stands for (kv_b's input), the rotary part unchanged."""
    from oracle import fp8
    e = np.array(entries, dtype=np.float64, copy=True)
    flat = e.reshape(-1, e.shape[-1])
    flat[:, :L] = fp8.quant_dequant_act(flat[:, :L])
    return flat.reshape(e.shape)
