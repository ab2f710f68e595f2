"""Build libmla.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m head_latent_attention_fwd_amd.build   (or build() from Python).
Every source is compiled on each call; objects go to _build/ next to csrc/.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmla.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")

SOURCES = ["api.cpp", "gemm_bf16.hip", "gemm_f32.hip", "gemm_fp8.hip", "gemm_skinny.hip", "elementwise.hip",
           "attn_prefill.hip", "attn_decode.hip", "decode_absorb.hip"]

# Packed-fp32 instructions stay off: ordinary float code is compiled to
# scalar VALU ops only.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libmla.so)")
    return p


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and "hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, errs in results:
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
