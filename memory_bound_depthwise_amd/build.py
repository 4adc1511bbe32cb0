"""Compile the HIP library libwtconv.so for gfx950, in-tree.

    python -m memory_bound_depthwise_amd.build

Flags: wave64 gfx950 code object, -O3, packed-FP32 instruction selection turned
off (plain v_fma_f32 only), host code C++17.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwtconv.so")
SOURCES = [os.path.join(CSRC, "wtconv_api.hip")]
HEADERS = [os.path.join(CSRC, "wtconv_kernels.hpp"), os.path.join(INCLUDE, "wtconv.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra_flags or []) + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libwtconv.so")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
