"""Compile the HIP library in-tree: swin3d_window_attention_amd/libswin3d_wattn.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libswin3d_wattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

ARCH = "gfx950"
# Packed FP32 instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def kernel_sources():
    """Every HIP source of the library, one kernel family per file."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile every source, link the shared library, and return its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    api_o = os.path.join(BUILD, "api.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c",
          os.path.join(CSRC, "api.cpp"), "-o", api_o], verbose)
    objs = [api_o]
    for src in kernel_sources():
        obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
