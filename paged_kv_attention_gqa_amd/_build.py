"""Compile libpkv.so for gfx950 in the package directory with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
SOURCES = ["csrc/api.cpp", "csrc/plan.cpp", "csrc/decode.hip", "csrc/mla.hip",
           "csrc/append.hip"]

# gfx950 only. Packed-fp32 VALU ops stay disabled; the kernels use MFMA and
# scalar fp32 only.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libpkv")
    return path


def build(verbose: bool = False) -> str:
    """Build (always, from source) and return the path of libpkv.so."""
    srcs = [os.path.join(PKG_DIR, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed building libpkv.so:\n" + " ".join(cmd))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
