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
    (1000, 136, 100003, "bf16"),   # 320x256 tile (16x16 MFMAs): ragged rows, vocabulary and K
    (4096, 64, 65536, "bf16"),     # 320x256 tile with the XCD remap, one k-stage per tile, ragged vocabulary
    (3000, 64, 120000, "bf16"),    # 320x256 tile without the XCD remap, ragged rows
    (3000, 64, 30000, "bf16"),     # 384x256 tile (32x32 MFMAs) with the XCD remap, ragged rows and vocabulary
    (1, 4, 1, "fp32"),
    (5, 36, 300, "fp32"),
    (257, 128, 1025, "fp32"),
]

# (N, D, V) for the tile- and chunk-boundary target test, one per tile size
BOUNDARY_SHAPES = [(512, 256, 50257), (1024, 64, 151936), (3000, 64, 30000)]



# ------------------------------------------------------------------ backward
# Tolerance for the backward, derived from its arithmetic: dZ = g p - g [v == y]
# is rounded once to the input dtype (unit roundoff u: 2^-8 for bf16, 2^-24 for
# fp32), and p = exp(z - lse) carries the fp32 error of z and of the forward's
# lse (an absolute error e in z - lse is a relative error e in p; 2e-5 is
# allowed, the bf16 forward's lse tolerance being 2e-3 and its measured errors
# ~5e-4 at |lse| ~ 366). Then each output is an fp32 sum of K terms. With S =
# sum over the terms of |g| (p + [v == y]) |other factor| (returned by the
# oracle), the error is at most (u + 2e-5) * S plus, for the fp32 sum, about
# sqrt(K) * 2^-24 * S with random rounding signs; the allowance takes four times
# that.
UNIT_ROUNDOFF = {torch.float32: 2.0 ** -24, torch.bfloat16: 2.0 ** -8}


def bwd_bound(abs_sum, dtype, K):
    u = UNIT_ROUNDOFF[dtype] + 2e-5
    return (u + 4.0 * np.sqrt(K) * 2.0 ** -24) * np.asarray(abs_sum, dtype=np.float64) + 1e-30


# Norm-wise, over all elements of one output: the errors that rounding dZ puts
# into the terms are u |term| at most and pseudo-random in sign and size (their
# root mean square is about u / sqrt(6) for round-to-nearest in a binary
# format), so they add up like the terms themselves when those carry random
# signs and less when one term dominates: ||error|| is about 0.4 u ||result||,
# and NORM_C = 1 asserts ||error|| <= u ||result|| (a margin of ~2.5). The
# error of p (2e-5 relative, the same for a whole row, so it does not average
# out) and the fp32 sums are bounded by the norm of the sums of |terms| S.
NORM_C = 1.0


def bwd_norm_bound(want, abs_sum, dtype, K):
    u = UNIT_ROUNDOFF[dtype]
    return (NORM_C * u * float(np.linalg.norm(want))
            + (2e-5 + 4.0 * np.sqrt(K) * 2.0 ** -24) * float(np.linalg.norm(abs_sum)) + 1e-30)


def check_bwd(got, want, abs_sum, dtype, K, what):
    """Elementwise (bwd_bound) and norm-wise (bwd_norm_bound) checks of one
    gradient; returns (max |d|, ||d|| / ||want||)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    err = np.abs(got - want)
    bound = bwd_bound(abs_sum, dtype, K)
    if not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: element {np.unravel_index(i, got.shape)}: got {got.flat[i]!r}, "
                             f"oracle {want.flat[i]!r}, |d|={err.flat[i]:.3e} > {bound.flat[i]:.3e}")
    del bound
    enorm = float(np.linalg.norm(err))
    nb = bwd_norm_bound(want, abs_sum, dtype, K)
    wnorm = float(np.linalg.norm(want))
    rel = enorm / wnorm if wnorm > 0 else float("nan")
    assert enorm <= nb, f"{what}: ||d|| = {enorm:.3e} > {nb:.3e} (relative {rel:.3e})"
    return float(err.max()) if err.size else 0.0, rel


def gpu_backward(H, W, y, g):
    """Forward (for lse), then the backward; returns dH, dW on the host."""
    import linear_cross_entropy_amd as flce
    _, lse = flce.flce_forward(H, W, y)
    dH, dW = flce.flce_backward(H, W, y, lse, g)
    torch.cuda.synchronize()
    return dH.cpu().numpy(), dW.cpu().numpy()


def parity_backward(H, W, y, g, what=""):
    """GPU backward against the oracle over every row and vocabulary entry."""
    dH, dW = gpu_backward(H, W, y, g)
    ref = oracle.backward(H.cpu(), W.cpu(), y.cpu(), g.cpu())
    N, D = H.shape
    V = W.shape[0]
    eh, rh = check_bwd(dH, ref["dH"], ref["dH_abs"], H.dtype, V, f"{what} dH")
    ew, rw = check_bwd(dW, ref["dW"], ref["dW_abs"], H.dtype, max(N, 1), f"{what} dW")
    return dH, dW, (eh, rh, ew, rw)


# (N, D, V, dtype) for the backward's full-parity grid: ragged rows, ragged
# vocabulary, partial last k-stages, several row chunks are not reachable at
# these sizes (one chunk), each tile size of the products.
BWD_SHAPES = [
    (1, 8, 1, "bf16"),
    (3, 72, 31, "bf16"),
    (257, 64, 1000, "bf16"),
    (300, 4104, 513, "bf16"),
    (512, 256, 32001, "bf16"),
    (1000, 136, 5003, "bf16"),
    (5, 36, 300, "fp32"),
    (257, 128, 1025, "fp32"),
]
