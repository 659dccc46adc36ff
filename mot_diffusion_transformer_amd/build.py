"""Build the HIP library libwam.so in-tree for gfx950 (cross-compiles without a GPU).

    python -m mot_diffusion_transformer_amd.build

Every call recompiles every source (parallel hipcc processes), then links
``mot_diffusion_transformer_amd/libwam.so``.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwam.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["misc.hip", "gemm.hip", "attention.hip", "wam_api.hip"]
# per-source extra flags: keep the attention's MFMA accumulators in VGPRs, so
# the softmax rescale works on them in place instead of copying to/from AGPRs;
# start every GEMM kernel on a 4 KB boundary (measured on MI355X: the video
# expert's tiled GEMMs ran up to ~2% slower at some offsets in the code
# object, with identical instructions, whenever other kernels changed size)
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "gemm.hip": ["-falign-functions=4096"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    warn = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line and line.strip())
    if warn.strip():
        sys.stderr.write(warn[-4000:] + "\n")
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
