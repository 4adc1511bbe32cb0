"""Build the CPU oracle (plain C, gcc, OpenMP) into oracle/libwtconv_oracle.so.

Test infrastructure: compiled by ``__graft_entry__.build()`` so the checker
exists wherever the tests run; never linked into the GPU library.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "wtconv_oracle.c")
OUT = os.path.join(_HERE, "libwtconv_oracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = OUT) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
