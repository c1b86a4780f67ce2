"""GPU parity of the backward (gradient of sum_i g_i loss_i wrt H and W)
against the float64 oracle, through the C ABI.

The tolerance is derived from the arithmetic (tests/parity.py: bwd_bound):
dZ is rounded once to the input dtype, then summed in fp32; the bound is that
rounding times the sum of the absolute values of each output's terms, which
the oracle returns alongside every output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import BWD_SHAPES, bwd_bound, check_bwd, check_close, gpu_backward, parity_backward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401


def _log(msg):
    print(msg, flush=True)


def _grad(N, seed, zeros=True):
    gen = torch.Generator().manual_seed(seed)
    g = torch.rand(N, generator=gen) * 2 - 0.5
    if zeros and N > 2:
        g[1] = 0.0
    return g.to(torch.float32).to(DEV)


@pytest.mark.parametrize("N,D,V,dt", BWD_SHAPES, ids=lambda v: str(v))
def test_backward_parity(N, D, V, dt):
    _log(f"[bwd] N={N} D={D} V={V} {dt}")
    std = 1.0 if dt == "bf16" else 0.5
    H, W, y = workloads.make_custom(N, D, V, dt, seed=N * 13 + V, device=DEV, h_std=std,
                                    w_std=0.5 / math.sqrt(D) * 4)
    g = _grad(N, seed=N + V)
    _, _, (eh, rh, ew, rw) = parity_backward(H, W, y, g, what=f"bwd N={N} D={D} V={V} {dt}")
    _log(f"[bwd] max |d| dH {eh:.3e} (rel {rh:.2e}), dW {ew:.3e} (rel {rw:.2e})")


def test_backward_out_of_range_target_and_zero_grad_rows():
    """A target outside [0, V) contributes g_i softmax(Z_i); g_i = 0 rows
    contribute nothing."""
    N, D, V = 64, 128, 1000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=5, device=DEV)
    y[0] = -1
    y[3] = V
    g = _grad(N, seed=9)
    g[5] = 0.0
    dH, dW, _ = parity_backward(H, W, y, g, what="bwd out-of-range targets")
    assert np.all(dH[5] == 0.0) and np.all(dH[1] == 0.0)


def test_backward_deterministic_bits():
    N, D, V = 512, 256, 50257
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=17, device=DEV)
    g = _grad(N, seed=3)
    a = gpu_backward(H, W, y, g)
    b = gpu_backward(H, W, y, g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_backward_production_shape_sparse_gradient():
    """Full production shape (N=8192, D=4096, V=151936, bf16), in the launch
    configuration the benchmark times, with the upstream gradient nonzero on 12
    rows only: then dW is the sum over those rows alone, which the oracle
    computes exactly on the sub-problem, and every other row of dH is 0."""
    w = workloads.WORKLOADS["prod_bf16"]
    _log(f"[bwd] {w.describe()} sparse gradient")
    H, W, y = workloads.make(w, DEV)
    rows = np.sort(workloads.subset_rows(w.N, 12, seed=99).numpy())
    g = torch.zeros(w.N, dtype=torch.float32)
    g[torch.as_tensor(rows)] = torch.linspace(0.25, 1.5, len(rows))
    g = g.to(DEV)
    dH, dW = gpu_backward(H, W, y, g)
    sel = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.backward(H.cpu()[sel], W.cpu(), y.cpu()[sel], g.cpu()[sel])
    check_bwd(dH[rows], ref["dH"], ref["dH_abs"], H.dtype, w.V, "prod dH rows")
    others = np.setdiff1d(np.arange(w.N), rows)
    assert np.all(dH[others] == 0.0), "rows with zero upstream gradient have nonzero dH"
    e, rel = check_bwd(dW, ref["dW"], ref["dW_abs"], H.dtype, w.N, "prod dW")
    _log(f"[bwd] prod dW max |d| {e:.3e}, relative Frobenius error {rel:.2e}")


def test_backward_production_shape_identities():
    """Dense upstream gradient at the production shape: sampled rows of dH
    against the oracle row by row, and on all of dW the identities
    sum_v dW_v = 0 and <dH, H> = <dW, W> (both hold exactly in real arithmetic)."""
    w = workloads.WORKLOADS["prod_bf16"]
    H, W, y = workloads.make(w, DEV)
    g = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=DEV)
    import linear_cross_entropy_amd as flce
    _, lse = flce.flce_forward(H, W, y)
    dH, dW = flce.flce_backward(H, W, y, lse, g)
    torch.cuda.synchronize()
    rows = workloads.subset_rows(w.N, 24, seed=5).numpy()
    ref = oracle.backward(H.cpu(), W.cpu(), y.cpu(), g.cpu(), rows=rows, want_dW=False)
    check_bwd(dH[torch.as_tensor(rows, device=DEV)].cpu().numpy(), ref["dH"], ref["dH_abs"], H.dtype, w.V,
              "prod dH sampled rows")
    # sum over the vocabulary of dW vanishes up to rounding: bound it by the
    # column sums of |dW| times the dZ rounding (each term's error is bounded
    # by u |term|, and |dW_vd| <= sum of |terms|)
    colsum = dW.double().sum(dim=0)
    colabs = dW.double().abs().sum(dim=0)
    assert bool((colsum.abs() <= 0.05 * colabs).all()), "sum_v dW_v is not ~0"
    ip_h = float((dH.double() * H.double()).sum())
    ip_w = float((dW.double() * W.double()).sum())
    scale = float((dH.double() * H.double()).abs().sum())
    assert abs(ip_h - ip_w) <= 2.0 ** -7 * scale, f"<dH,H>={ip_h} vs <dW,W>={ip_w} (scale {scale})"
    _log(f"[bwd] prod identities: <dH,H>={ip_h:.6e} <dW,W>={ip_w:.6e}")


@pytest.mark.parametrize("name", ["small_bf16", "medium_bf16"])
def test_backward_vocabulary_split_workloads(name):
    """The small and medium bf16 workloads, whose dH product has too few tiles
    to fill the chip and is split over the vocabulary into partial sums (the
    workspace is larger than W^T, H^T and dZ^T alone). Dense upstream gradient
    1/N: sampled rows of dH against the oracle row by row; for the small
    workload all of dW too; and the same bits on a second call."""
    import linear_cross_entropy_amd as flce
    w = workloads.WORKLOADS[name]
    _log(f"[bwd] {w.describe()} vocabulary split")
    up = lambda x: (x + 63) // 64 * 64
    base = sum((n * 2 + 255) // 256 * 256 for n in (w.D * up(w.V), w.D * up(w.N), up(w.V) * up(w.N)))
    assert flce.flce_backward_workspace_bytes(w.N, w.D, w.V, "bf16") > base
    H, W, y = workloads.make(w, DEV)
    g = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=DEV)
    _, lse = flce.flce_forward(H, W, y)
    dH, dW = flce.flce_backward(H, W, y, lse, g)
    dH2, dW2 = flce.flce_backward(H, W, y, lse, g)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2), "second call differs"
    rows = workloads.subset_rows(w.N, 24, seed=11).numpy()
    full = name == "small_bf16"
    ref = oracle.backward(H.cpu(), W.cpu(), y.cpu(), g.cpu(), rows=None if full else rows, want_dW=full)
    ref_dH = ref["dH"][rows] if full else ref["dH"]
    ref_abs = ref["dH_abs"][rows] if full else ref["dH_abs"]
    check_bwd(dH[torch.as_tensor(rows, device=DEV)].cpu().numpy(), ref_dH, ref_abs, H.dtype, w.V,
              f"{name} dH sampled rows")
    if full:
        e, rel = check_bwd(dW.cpu().numpy(), ref["dW"], ref["dW_abs"], H.dtype, w.N, f"{name} dW")
        _log(f"[bwd] {name} dW max |d| {e:.3e}, relative Frobenius error {rel:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_ragged_rows_and_vocabulary_slices(dtype):
    """N=5000, V=262144 with the upstream gradient on a few rows (the others
    must get dH = 0). The dZ budget splits the vocabulary into slices: bf16
    three of up to 92160 rows (dZ read transposed for dH), fp32 eleven of up
    to 24576 (row-major dZ); dH adds up the slices' products in place. The
    gradient rows' targets sit on both sides of every slice boundary. All of
    dW and the gradient rows of dH against the oracle on those rows."""
    import linear_cross_entropy_amd as flce
    N, D, V = 5000, 64, 262144
    vs = 92160 if dtype == "bf16" else 24576
    assert flce.flce_backward_workspace_bytes(N, D, V, dtype) > 0
    H, W, y = workloads.make_custom(N, D, V, dtype, seed=21, device=DEV)
    bounds = [b for k in range(1, -(-V // vs)) for b in (k * vs - 1, k * vs)]
    rows = np.unique(np.concatenate([np.array([0, 7, 2559, 2560, 4991, 4999]),
                                     np.linspace(8, 4990, len(bounds)).astype(np.int64)]))
    tgt = np.array((bounds + [0, V - 1] * len(rows))[:len(rows)], dtype=np.int32)
    y[torch.as_tensor(rows, device=DEV)] = torch.as_tensor(tgt, device=DEV)
    g = torch.zeros(N, dtype=torch.float32)
    g[torch.as_tensor(rows)] = torch.linspace(0.5, 1.25, len(rows))
    g = g.to(DEV)
    dH, dW = gpu_backward(H, W, y, g)
    sel = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.backward(H.cpu()[sel], W.cpu(), y.cpu()[sel], g.cpu()[sel])
    check_bwd(dH[rows], ref["dH"], ref["dH_abs"], H.dtype, V, f"{dtype} dH rows")
    assert np.all(dH[np.setdiff1d(np.arange(N), rows)] == 0.0)
    check_bwd(dW, ref["dW"], ref["dW_abs"], H.dtype, N, f"{dtype} dW")


def test_backward_stress_shape_sparse_gradient():
    """The large-vocabulary stress workload (N=8192, D=8192, V=262144, 64
    outlier W rows). Gradient on 8 rows spread over the batch; all of dW and
    those dH rows against the oracle on those rows."""
    w = workloads.WORKLOADS["stress_bf16"]
    _log(f"[bwd] {w.describe()} sparse gradient")
    H, W, y = workloads.make(w, DEV)
    rows = np.array([0, 1500, 2815, 2816, 5000, 5631, 5632, 8191])
    g = torch.zeros(w.N, dtype=torch.float32)
    g[torch.as_tensor(rows)] = torch.linspace(0.25, 2.0, len(rows))
    g = g.to(DEV)
    dH, dW = gpu_backward(H, W, y, g)
    sel = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.backward(H.cpu()[sel], W.cpu(), y.cpu()[sel], g.cpu()[sel])
    check_bwd(dH[rows], ref["dH"], ref["dH_abs"], H.dtype, w.V, "stress dH rows")
    assert np.all(dH[np.setdiff1d(np.arange(w.N), rows)] == 0.0)
    worst = 0.0
    for v0 in range(0, w.V, 16384):       # blocks of vocabulary rows keep host temporaries small
        e, _ = check_bwd(dW[v0:v0 + 16384], ref["dW"][v0:v0 + 16384], ref["dW_abs"][v0:v0 + 16384],
                         H.dtype, w.N, f"stress dW rows {v0}..")
        worst = max(worst, e)
    _log(f"[bwd] stress dW max |d| {worst:.3e}")


def test_backward_medium_workload_sparse_gradient():
    """The medium workload (N=4096, D=2048, V=50257, Zipf targets; dH split
    over the vocabulary) with the upstream gradient on 16 rows, among them
    rows whose targets are the most frequent word: all of dW (the oracle
    computes it exactly on those rows alone, the others' dZ being 0) and those
    rows of dH against the oracle, every other dH row exactly 0."""
    w = workloads.WORKLOADS["medium_bf16"]
    _log(f"[bwd] {w.describe()} sparse gradient")
    H, W, y = workloads.make(w, DEV)
    yc = y.cpu().numpy()
    top = np.nonzero(yc == np.bincount(yc).argmax())[0][:4]
    rows = np.unique(np.concatenate([top, workloads.subset_rows(w.N, 12, seed=31).numpy()]))
    g = torch.zeros(w.N, dtype=torch.float32)
    g[torch.as_tensor(rows)] = torch.linspace(-0.75, 1.5, len(rows))
    g = g.to(DEV)
    dH, dW = gpu_backward(H, W, y, g)
    sel = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.backward(H.cpu()[sel], W.cpu(), y.cpu()[sel], g.cpu()[sel])
    eh, rh = check_bwd(dH[rows], ref["dH"], ref["dH_abs"], H.dtype, w.V, "medium dH rows")
    assert np.all(dH[np.setdiff1d(np.arange(w.N), rows)] == 0.0)
    ew, rw = check_bwd(dW, ref["dW"], ref["dW_abs"], H.dtype, w.N, "medium dW")
    _log(f"[bwd] medium dH max |d| {eh:.3e} rel {rh:.2e}; dW max |d| {ew:.3e} rel {rw:.2e}")


def test_buffers_beyond_two_gib():
    """H of 2 GiB (N = 131072, D = 8192 bf16) and a 4 GiB dH: the last rows of H
    start beyond 2^31 bytes and those of dH beyond 2^32, so every row offset
    must be computed in 64 bits (the buffer resources are made per row block).
    Forward on sampled rows including the last ones; backward with the
    gradient on 10 rows spread over the batch: those dH rows and all of dW
    against the oracle, every other dH row exactly 0 (checked on the GPU)."""
    import linear_cross_entropy_amd as flce
    N, D, V = 131072, 8192, 4000
    _log(f"[big buffers] N={N} D={D} V={V} bf16")
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=2031, device=DEV, h_std=1.0, w_std=1.0 / D ** 0.5)
    assert H.numel() * H.element_size() >= 2 ** 31
    rows = np.array([0, 1, 255, 256, 65535, 65536, 131000, 131069, 131070, 131071])
    y[torch.as_tensor(rows[-4:], device=DEV)] = torch.tensor([0, V - 1, 1234, V - 2], dtype=torch.int32, device=DEV)
    loss, lse = flce.flce_forward(H, W, y)
    torch.cuda.synchronize()
    Hc, Wc, yc = H.cpu(), W.cpu(), y.cpu()
    rl, rs, _ = oracle.forward(Hc, Wc, yc, rows=rows)
    check_close(lse.cpu().numpy()[rows], rs, H.dtype, "big buffers lse")
    check_close(loss.cpu().numpy()[rows], rl, H.dtype, "big buffers loss")
    g = torch.zeros(N, dtype=torch.float32)
    g[torch.as_tensor(rows)] = torch.linspace(0.5, 1.5, len(rows))
    g = g.to(DEV)
    dH, dW = flce.flce_backward(H, W, y, lse, g)
    torch.cuda.synchronize()
    assert dH.numel() * dH.element_size() >= 2 ** 32
    mask = torch.ones(N, dtype=torch.bool, device=DEV)
    mask[torch.as_tensor(rows, device=DEV)] = False
    assert bool((dH[mask] == 0).all().item()), "dH nonzero off the gradient rows"
    sel = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.backward(Hc[sel], Wc, yc[sel], g.cpu()[sel])
    check_bwd(dH[sel.to(DEV)].cpu().numpy(), ref["dH"], ref["dH_abs"], H.dtype, V, "big buffers dH rows")
    e, rel = check_bwd(dW.cpu().numpy(), ref["dW"], ref["dW_abs"], H.dtype, N, "big buffers dW")
    _log(f"[big buffers] dW max |d| {e:.3e}, relative Frobenius error {rel:.2e}")
