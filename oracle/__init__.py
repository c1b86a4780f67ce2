"""Oracle for the fused linear cross-entropy forward and backward -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. It is a plain float64 CPU
implementation of the definition on the page "Een gefuseerde forward-kernel
voor lineaire cross-entropy op Apple-GPU's" (section 1): Z = H W^T and
loss_i = logsumexp(Z_i) - Z_{i, y_i}, and the gradient of sum_i g_i loss_i
with respect to H and W (the chain rule on that definition). The arithmetic lives in
``flce_oracle.c`` (plain C, OpenMP over rows); this module only builds it and
marshals arguments. It shares no code with the GPU library.

Pins (what ties it to something other than itself) are the ``not gpu`` tests
in ``tests/test_oracle_pins.py`` and ``tests/test_oracle_mutants.py``.

``dequantize`` writes out the quantised-head format the library takes for
the page's quantised output heads (section 2 mentions them; no format is
fixed there, so the format is a reading, stated with the library's
flce_forward_quant): it is pinned by closed forms in
``tests/test_oracle_quant.py``, while the choice of format itself has
nothing on the page to be checked against (parity unpinned in that sense).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flce_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load the oracle library, building it first if nothing is built."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    lib.oracle_lce_forward.restype = ctypes.c_int
    lib.oracle_lce_forward.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_lce_backward.restype = ctypes.c_int
    lib.oracle_lce_backward.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _as_numpy(x):
    """Host array with the exact bits of x: bf16 -> uint16, fp32 -> float32."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), 0
            if x.dtype == torch.float32:
                return x.numpy(), 1
            if x.dtype == torch.int32:
                return x.numpy(), None
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 0
    if x.dtype == np.float32:
        return x, 1
    if x.dtype == np.int32:
        return x, None
    raise TypeError(f"unsupported dtype {x.dtype}")


def num_threads() -> int:
    return int(load().oracle_num_threads())


def forward(H, W, y, rows=None, lib=None):
    """Return (loss, lse, z_target) as float64 numpy arrays.

    H: (N, D), W: (V, D), both bfloat16 or both float32 (torch CPU/GPU
    tensors, or numpy uint16 bit patterns / float32); y: int32 (N).
    rows: optional sequence of row indices; outputs follow that order.
    """
    lib = lib or load()
    h, dt_h = _as_numpy(H)
    w, dt_w = _as_numpy(W)
    t, _ = _as_numpy(y)
    if dt_h != dt_w or dt_h is None:
        raise TypeError("H and W must share a floating dtype")
    if t.dtype != np.int32:
        raise TypeError("targets must be int32")
    N, D = h.shape
    V, D2 = w.shape
    if D2 != D or t.shape != (N,):
        raise ValueError("shape mismatch")
    if rows is None:
        R = N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_arr.shape[0]
    loss = np.empty(R, np.float64)
    lse = np.empty(R, np.float64)
    zt = np.empty(R, np.float64)
    rc = lib.oracle_lce_forward(
        h.ctypes.data, w.ctypes.data, t.ctypes.data, N, D, V, dt_h,
        rows_arr.ctypes.data if rows_arr is not None else None, R,
        loss.ctypes.data, lse.ctypes.data, zt.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return loss, lse, zt


def backward(H, W, y, g, rows=None, want_dW=True, lib=None):
    """Gradient of sum_i g_i loss_i: returns a dict of float64 arrays
    dH (R, D) and dH_abs for the selected rows (all rows if rows is None), and,
    when want_dW, dW (V, D) and dW_abs over all rows. The *_abs arrays are the
    sums of the absolute values of each output's terms, with dZ split into its
    two terms g p and -g [v == y] (so V = 1, where dZ = 0, still has a size).

    g: the upstream gradient per token (float32 or float64, length N); it is
    widened exactly to float64.
    """
    lib = lib or load()
    h, dt_h = _as_numpy(H)
    w, dt_w = _as_numpy(W)
    t, _ = _as_numpy(y)
    if dt_h != dt_w or dt_h is None:
        raise TypeError("H and W must share a floating dtype")
    if t.dtype != np.int32:
        raise TypeError("targets must be int32")
    try:
        import torch
        if isinstance(g, torch.Tensor):
            g = g.detach().cpu().numpy()
    except ImportError:
        pass
    gd = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
    N, D = h.shape
    V, D2 = w.shape
    if D2 != D or t.shape != (N,) or gd.shape != (N,):
        raise ValueError("shape mismatch")
    if rows is None:
        R, rows_arr = N, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_arr.shape[0]
    dH = np.empty((R, D), np.float64)
    dH_abs = np.empty((R, D), np.float64)
    dW = np.empty((V, D), np.float64) if want_dW else None
    dW_abs = np.empty((V, D), np.float64) if want_dW else None
    rc = lib.oracle_lce_backward(
        h.ctypes.data, w.ctypes.data, t.ctypes.data, gd.ctypes.data, N, D, V, dt_h,
        rows_arr.ctypes.data if rows_arr is not None else None, R,
        dH.ctypes.data, dH_abs.ctypes.data,
        dW.ctypes.data if want_dW else None, dW_abs.ctypes.data if want_dW else None)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"dH": dH, "dH_abs": dH_abs}
    if want_dW:
        out["dW"] = dW
        out["dW_abs"] = dW_abs
    return out


def _bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), rounding to nearest,
    ties to even (inputs here are finite)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def dequantize(codes, scales, biases, bits: int, group: int) -> np.ndarray:
    """bf16 bit patterns (uint16, V x D) of the quantised head
    w[v][d] = bf16(fl32(fl32(scale[v][d // group] * q[v][d]) + bias[v][d // group])).

    codes: uint8, V x D (bits = 8) or V x D/2 (bits = 4: byte b holds q of
    weight 2b in its low nibble, of 2b + 1 in its high nibble); scales and
    biases: float32, V x (D / group). Step by step as the formula reads: the
    codes as float32, one float32 product, one float32 sum, one rounding to
    bf16.
    """
    c = np.asarray(codes.cpu() if hasattr(codes, "cpu") else codes, dtype=np.uint8)
    sc = np.asarray(scales.cpu() if hasattr(scales, "cpu") else scales, dtype=np.float32)
    bi = np.asarray(biases.cpu() if hasattr(biases, "cpu") else biases, dtype=np.float32)
    if bits == 8:
        q = c
    elif bits == 4:
        q = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.uint8)
        q[:, 0::2] = c & 0x0F
        q[:, 1::2] = c >> 4
    else:
        raise ValueError("bits must be 4 or 8")
    V, D = q.shape
    if group <= 0 or D % group or sc.shape != (V, D // group) or bi.shape != (V, D // group):
        raise ValueError("group must divide D; scales and biases must be V x D/group")
    s_full = np.repeat(sc, group, axis=1)
    b_full = np.repeat(bi, group, axis=1)
    prod = q.astype(np.float32) * s_full          # float32 * float32 -> one rounding
    w32 = (prod + b_full).astype(np.float32)      # float32 + float32 -> one rounding
    return _bf16_rne_bits(w32)

