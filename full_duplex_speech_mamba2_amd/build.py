"""Build libm2.so in-tree with hipcc for gfx950.

    python -m full_duplex_speech_mamba2_amd.build

Packed-fp32 instructions are switched off for all device code
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libm2.so")
SOURCES = ["m2_api.cpp", "decode.hip", "fused.hip", "prefill.hip", "attention.hip"]
ARCH = os.environ.get("M2_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def build(verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "-c", path, "-o", obj, "--offload-arch=" + ARCH] + common
        if src.endswith(".cpp"):
            cmd = [hipcc(), "-x", "hip", "-c", path, "-o", obj, "--offload-arch=" + ARCH] + common
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + [
        "-Wl,-soname,libm2.so", "-Wl,-z,defs", "-L/opt/rocm/lib", "-lamdhip64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
