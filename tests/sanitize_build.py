"""Host-sanitized build of libsherry.so for the CPU tests.

The C ABI layer (abi.cpp: argument validation, plan building, dispatch) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host code
only; the kernels' objects are the regular ones (GPU code is never built with a
sanitizer).  tests/test_abi_sanitized.py runs the host ABI tests against the
result with the sanitizer runtime preloaded into the Python process.
"""
from __future__ import annotations

import glob
import os
import subprocess

from ultra_bit_weight_amd import build as b

# each sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The shared sanitizer runtime that hipcc's clang links against."""
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")) + \
        sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    if not cands:
        raise RuntimeError("clang's shared AddressSanitizer runtime not found under /opt/rocm/llvm")
    return cands[-1]


def build(out_dir: str) -> str:
    """Compile abi.cpp with the host sanitizers, link it with the regular
    kernel objects (built first if missing) into out_dir/libsherry_san.so."""
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in b.SOURCES:
        if src == "abi.cpp":
            continue
        obj = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            os.makedirs(b.BUILD, exist_ok=True)
            b._compile(src, False, b.BUILD, ())
        objs.append(obj)
    abi_o = os.path.join(out_dir, "abi_san.o")
    cmd = [b.hipcc(), *b.common_flags(), "-O1", "-g", *HOST_SAN, "-c", os.path.join(b.CSRC, "abi.cpp"), "-o", abi_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    out = os.path.join(out_dir, "libsherry_san.so")
    cmd = [b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libasan", "-o", out, abi_o,
           *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out
