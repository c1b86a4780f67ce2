"""Binding of libflce_ceiling.so: the sustained rate of the bf16 matrix-core
instruction the forward's contraction uses, with operands in registers and no
memory traffic, and the shader clock the part held meanwhile. A measuring
instrument (declared in include/flce_ceiling.h), not part of the forward.

    flce_ceiling_mfma(ops, order, iters, grid, threads=512, lds_bytes=0, stream=None)
        -> (out, clocks)   both device tensors; see the header for their meaning
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflce_ceiling.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python linear_cross_entropy_amd/_build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_lib.flce_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.flce_ceiling_mfma.restype = ctypes.c_int

FLOP_PER_MFMA = 32 * 32 * 16 * 2
MFMA_PER_ITER = 32


def flce_ceiling_mfma(ops: torch.Tensor, order: int, iters: int, grid: int, threads: int = 512,
                      lds_bytes: int = 0, stream=None):
    if ops.dtype != torch.bfloat16 or not ops.is_cuda or not ops.is_contiguous():
        raise ValueError("ops must be a contiguous bf16 CUDA tensor")
    if ops.numel() < grid * threads * 64:
        raise ValueError(f"ops needs {grid * threads * 64} elements (8 fragments of 8 per thread)")
    out = torch.empty(grid * threads, dtype=torch.float32, device=ops.device)
    clocks = torch.zeros(grid * 4, dtype=torch.int64, device=ops.device)
    s = stream if stream is not None else torch.cuda.current_stream(ops.device)
    rc = _lib.flce_ceiling_mfma(ctypes.c_void_p(ops.data_ptr()), order, iters, grid, threads, lds_bytes,
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                                ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"flce_ceiling_mfma failed with status {rc}")
    return out, clocks
