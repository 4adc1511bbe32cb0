"""Compile the HIP library libwtconv.so for gfx950, in-tree.

    python -m memory_bound_depthwise_amd.build

The host side (C ABI, plans) is one translation unit; the kernels and launch
sequences are compiled once per kernel size and activation type from
csrc/wtconv_inst.hip (nine units, compiled in parallel) and linked with it.

Flags: wave64 gfx950 code object, -O3, packed-FP32 instruction selection turned
off (plain v_fma_f32 only), host code C++17, only the C interface exported.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwtconv.so")
API = os.path.join(CSRC, "wtconv_api.hip")
INST = os.path.join(CSRC, "wtconv_inst.hip")
KERNEL_SIZES = (3, 5, 7)
STORAGE = {"f32": "float", "bf16": "uint16_t", "f16": "wtc_f16"}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def units():
    """(source, extra defines, object stem) of every translation unit."""
    out = [(API, [], "api")]
    for k in KERNEL_SIZES:
        for name, ctype in STORAGE.items():
            out.append((INST, [f"-DWTC_K={k}", f"-DWTC_T={ctype}"], f"inst_k{k}_{name}"))
    return out


def _jobs():
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit():
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    extra = list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="wtconv_build_") as tmpdir:
        def compile_one(unit):
            src, defs, stem = unit
            obj = os.path.join(tmpdir, stem + ".o")
            cmd = [HIPCC] + FLAGS + extra + defs + ["-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return obj, res, cmd

        objs = []
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            for obj, res, cmd in pool.map(compile_one, units()):
                if res.returncode != 0:
                    sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
                    raise RuntimeError("hipcc failed to build libwtconv.so")
                if verbose and res.stderr.strip():
                    sys.stderr.write(res.stderr)
                objs.append(obj)
        tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
            raise RuntimeError("linking libwtconv.so failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
