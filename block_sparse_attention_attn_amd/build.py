"""Build libvsa.so (the gfx950 HIP kernels plus the C-ABI entry points) in-tree.

    python -m block_sparse_attention_attn_amd.build

Compiles every ``csrc/*.hip`` with ``hipcc --offload-arch=gfx950`` into ``_build/`` (in
parallel) and links ``block_sparse_attention_attn_amd/libvsa.so``. Packed-FP32 instruction
selection is switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libvsa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libvsa.so")


FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source code generation options. The backward kernels keep their MFMA accumulators in
# VGPRs, where the softmax arithmetic reads them, instead of accumulation registers that would
# need a copy per element per step.
SOURCE_FLAGS = {
    "bwd_dkdv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_dq_spill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(" ".join(cmd))
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link; returns the path of libvsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
