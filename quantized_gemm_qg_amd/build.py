"""Build libqg.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python quantized_gemm_qg_amd/build.py

Every source compiles to its own object (in parallel), then links into
``quantized_gemm_qg_amd/libqg.so``.  Packed-fp32 VALU instructions are disabled
for device code (``-packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqg.so")
SOURCES = ["qg_api.cpp", "qg_repack.cpp", "qg_kernels.hip", "qg_formats.hip", "qg_tiled.hip", "qg_tiled_a16.hip",
           "qg_act.hip"]
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
    ]


# Per-source extra flags.  The integer-format tiled kernel keeps its MFMA
# results in VGPRs (they feed fp32 FMAs right away); left to its heuristics the
# compiler puts them in AGPRs and copies every one back.
EXTRA = {"qg_tiled_a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", *_flags(), *EXTRA.get(src, []), "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libqg.so; returns its path.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
