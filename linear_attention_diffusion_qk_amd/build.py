"""Build libsanala.so in-tree for gfx950 with hipcc (no JIT, no torch extension machinery).

    python -m linear_attention_diffusion_qk_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsanala.so")
SOURCES = ["attn_plan.hip", "attn_f32.hip", "attn_bf16.hip", "kv_state_x.hip", "gemm_kernel.hip", "mix_ffn.hip", "cross_attn.hip", "sanala_api.hip"]
ARCH = os.environ.get("SANA_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 VALU instructions are kept out of the device code on purpose.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result",
]

# Per-source additions.  The cross-attention's softmax reads every MFMA result on the vector ALU, so its
# accumulators are kept in ordinary VGPRs (with the compiler's choice, AGPRs, each result crossed over by
# an extra move; the kernel went from 98 VGPR + 24 AGPR with 176 moves to 98 VGPR and none).  The GEMMs
# keep the default: their 192 accumulators per lane need the AGPR file.
EXTRA_FLAGS = {"cross_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libsanala needs ROCm's hipcc to build")
    return exe


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libsanala.so next to this file; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPFLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = _run(cmd)
        # The host pass does not know the packed-fp32 target feature and says so; anything else is shown.
        warn = [ln for ln in (r.stderr or "").splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
        if warn:
            print(f"{src}:\n" + "\n".join(warn), flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
