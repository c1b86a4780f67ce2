"""The autograd op linear_cross_entropy: its loss and the gradients autograd
delivers to H and W must be exactly those of flce_forward and flce_backward
called directly with the same per-token upstream gradient (bf16 inputs get the
float32 gradients cast to bf16 by autograd), and match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_bwd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_autograd_matches_the_direct_calls(dt):
    import linear_cross_entropy_amd as flce
    N, D, V = (777, 256, 9001) if dt == "bf16" else (130, 64, 1500)
    print(f"[autograd] N={N} D={D} V={V} {dt}", flush=True)
    H0, W0, y = workloads.make_custom(N, D, V, dt, seed=53, device=DEV)
    weights = torch.linspace(-1.0, 2.0, N, dtype=torch.float32, device=DEV)
    H = H0.clone().requires_grad_(True)
    W = W0.clone().requires_grad_(True)
    loss = flce.linear_cross_entropy(H, W, y)
    (loss * weights).sum().backward()
    torch.cuda.synchronize()

    loss_d, lse_d = flce.flce_forward(H0, W0, y)
    dH_d, dW_d = flce.flce_backward(H0, W0, y, lse_d, weights.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(loss.detach(), loss_d)
    assert H.grad.dtype == H0.dtype and W.grad.dtype == W0.dtype
    assert torch.equal(H.grad, dH_d.to(H0.dtype))
    assert torch.equal(W.grad, dW_d.to(W0.dtype))


def test_autograd_mean_against_the_oracle():
    """Gradient of the mean loss (upstream 1/N per token) against the float64
    oracle, fp32 inputs (no rounding of the gradients afterwards)."""
    import linear_cross_entropy_amd as flce
    N, D, V = 200, 96, 3001
    H0, W0, y = workloads.make_custom(N, D, V, "fp32", seed=59, device=DEV, h_std=0.5,
                                      w_std=1.0 / np.sqrt(D))
    H = H0.clone().requires_grad_(True)
    W = W0.clone().requires_grad_(True)
    flce.linear_cross_entropy(H, W, y).mean().backward()
    torch.cuda.synchronize()
    g = torch.full((N,), 1.0 / N, dtype=torch.float32)
    ref = oracle.backward(H0.cpu(), W0.cpu(), y.cpu(), g)
    check_bwd(H.grad.cpu().numpy(), ref["dH"], ref["dH_abs"], H0.dtype, V, "autograd dH")
    check_bwd(W.grad.cpu().numpy(), ref["dW"], ref["dW_abs"], H0.dtype, N, "autograd dW")


def test_autograd_only_the_inputs_that_need_it():
    import linear_cross_entropy_amd as flce
    N, D, V = 64, 64, 700
    H0, W0, y = workloads.make_custom(N, D, V, "bf16", seed=61, device=DEV)
    H = H0.clone().requires_grad_(True)
    flce.linear_cross_entropy(H, W0, y).sum().backward()
    torch.cuda.synchronize()
    _, lse = flce.flce_forward(H0, W0, y)
    dH, _ = flce.flce_backward(H0, W0, y, lse, torch.ones(N, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert W0.grad is None
    assert torch.equal(H.grad, dH.to(H0.dtype))


def test_autograd_ignored_positions():
    """Targets of -100 on some rows: their loss is NaN, and reducing over the
    valid rows gives the gradients of those rows alone (the oracle on the
    valid sub-batch for dW; zero dH on the ignored rows)."""
    import linear_cross_entropy_amd as flce
    N, D, V = 300, 128, 4001
    H0, W0, y = workloads.make_custom(N, D, V, "fp32", seed=67, device=DEV, h_std=0.5,
                                      w_std=1.0 / np.sqrt(D))
    y = y.clone()
    y[::7] = -100
    H = H0.clone().requires_grad_(True)
    W = W0.clone().requires_grad_(True)
    loss = flce.linear_cross_entropy(H, W, y)
    valid = y >= 0
    assert bool(torch.isnan(loss[~valid]).all()) and bool(torch.isfinite(loss[valid]).all())
    loss[valid].sum().backward()
    torch.cuda.synchronize()
    assert bool((H.grad[~valid] == 0).all())
    sel = valid.cpu()
    ref = oracle.backward(H0.cpu()[sel], W0.cpu(), y.cpu()[sel], torch.ones(int(sel.sum()), dtype=torch.float32))
    check_bwd(H.grad.cpu().numpy()[sel.numpy()], ref["dH"], ref["dH_abs"], H0.dtype, V, "ignored rows: dH")
    check_bwd(W.grad.cpu().numpy(), ref["dW"], ref["dW_abs"], H0.dtype, N, "ignored rows: dW")
