"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle
on the same bits, compare to the stated tolerance.

Tolerances (stated for the benchmark workloads and used for every case):
  fp32 inputs: |gpu - oracle| <= 1e-5 * max(1, |oracle|)
  bf16 inputs: |gpu - oracle| <= 2e-3 (fp32 accumulation on both loss and lse)
NaN must match NaN position for position.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {torch.float32: ("rel", 1e-5), torch.bfloat16: ("abs", 2e-3)}


def check_close(got, want, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ at {np.nonzero(nan_g != nan_w)[0][:8]}"
    ok = ~nan_w
    kind, tol = TOL[dtype]
    err = np.abs(got[ok] - want[ok])
    bound = tol * np.maximum(1.0, np.abs(want[ok])) if kind == "rel" else np.full(err.shape, tol)
    if err.size and not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        idx = np.nonzero(ok)[0][i]
        raise AssertionError(f"{what}: row {idx}: got {got[idx]!r}, oracle {want[idx]!r}, "
                             f"|d|={err[i]:.3e} > {bound[i]:.3e}; max |d| {err.max():.3e}")
    return float(err.max()) if err.size else 0.0


def gpu_forward(H, W, y):
    import linear_cross_entropy_amd as flce
    loss, lse = flce.flce_forward(H, W, y)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy()


def parity(H, W, y, rows=None, what="", Hc=None, Wc=None):
    """GPU forward over all rows; the oracle on `rows` (all when None)."""
    loss, lse = gpu_forward(H, W, y)
    Hc = H.cpu() if Hc is None else Hc
    Wc = W.cpu() if Wc is None else Wc
    yc = y.cpu()
    rl, rs, _ = oracle.forward(Hc, Wc, yc, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    e1 = check_close(lse[sel], rs, H.dtype, f"{what} lse")
    e2 = check_close(loss[sel], rl, H.dtype, f"{what} loss")
    return loss, lse, max(e1, e2)


# Edge shapes for the GPU parity grid (N, D, V, dtype): degenerate sizes,
# ragged rows, vocabulary and K, and shapes large enough that the planner
# picks each tile configuration (a host-side test checks that all of them are
# exercised).
EDGE = [
    (1, 8, 1, "bf16"),
    (3, 8, 2, "bf16"),
    (3, 72, 31, "bf16"),
    (257, 72, 255, "bf16"),
    (257, 64, 256, "bf16"),
    (3, 64, 257, "bf16"),
    (300, 4104, 513, "bf16"),
    (64, 1024, 32001, "bf16"),
    (64, 1024, 31999, "bf16"),
    (40, 256, 50257, "bf16"),
    (1000, 136, 100003, "bf16"),   # 320x256 tile: ragged rows, vocabulary and K
    (4096, 64, 65536, "bf16"),     # 384x256 tile, one k-stage per tile, ragged vocabulary
    (3000, 64, 120000, "bf16"),    # 384x256 tile without the XCD remap, ragged rows and vocabulary
    (1, 4, 1, "fp32"),
    (5, 36, 300, "fp32"),
    (257, 128, 1025, "fp32"),
]

# (N, D, V) for the tile- and chunk-boundary target test, one per tile size
BOUNDARY_SHAPES = [(512, 256, 50257), (1024, 64, 151936), (4096, 64, 65536)]

