"""Build libsherry.so in-tree with hipcc for gfx950.

    python -m ultra_bit_weight_amd.build

Objects go to ultra_bit_weight_amd/_build/, the library to
ultra_bit_weight_amd/lib/libsherry.so (written atomically).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsherry.so")
SOURCES = ["abi.cpp", "pack.hip", "gemv.hip", "gemm.hip", "gemm_bf16.hip", "gemm_prefill.hip", "gemm_tile32.hip", "act.hip", "probes.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsherry.so)")


def common_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    ]


# Per-source flags.  gemm.hip and probes.hip: MFMA accumulators in ordinary
# VGPRs (the default AGPR form made the compiler copy the tiled kernel's
# accumulators between the two register files on every k step, and the rate
# probe's 4 products per iteration came with 20 such copies).
FILE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, save_temps: bool, objdir: str, defines) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *FILE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, save_temps: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source and link `out` (default: the in-tree library).
    `defines` (NAME=VALUE strings) override the build-time tunables."""
    tag = "_".join(d.replace("=", "") for d in defines)
    objdir = os.path.join(BUILD, tag) if tag else BUILD
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    srcs = list(SOURCES)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps, objdir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
