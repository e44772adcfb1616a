"""Build libwsp.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m video_dit_window_amd.build [-v]
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwsp.so")
ARCH = "gfx950"

SOURCES = ["plan.cpp", "abi.cpp", "relayout.hip", "rope.hip", "text_mean.hip", "attn_f32.hip",
           "attn_bf16.hip", "fp8.hip", "gemm_bf16.hip", "xcd_probe.hip"]

# Packed-FP32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwsp)")


# Per-source flags.  attn_bf16.hip: the resident work groups take their next
# ticket with one atomic from one lane; LLVM's atomic optimizer would rewrite
# it into a wave-wide form that reads the result back at once, i.e. waits for
# every outstanding memory operation (the previous item's output stores
# included) at the start of each item.
EXTRA_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS +
           EXTRA_FLAGS.get(src, []))
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libwsp.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libwsp.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
