"""Compile the HIP libraries in-tree for gfx950: libflce.so (the fused linear
cross-entropy) and libflce_ceiling.so (the matrix-core ceiling instrument)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "flce.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflce.so")
CEILING_SRC = os.path.join(PKG, "csrc", "ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libflce_ceiling.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled for every HIP translation unit.
# Floating-point contraction is off: the kernels write every FMA explicitly,
# and the online-softmax rescale relies on products being rounded on their own.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, out: str, extra: list[str] | None, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Build libflce.so (at `out`) and, beside the default library, the ceiling instrument."""
    _compile(SRC, out, extra, verbose)
    if out == LIB:
        _compile(CEILING_SRC, CEILING_LIB, None, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
