"""Seeded random shapes: forward, backward and the quantised head against the
oracle on every row.

The fixed grids in parity.py are chosen by hand for known edges; these shapes
are drawn once from a fixed seed over wide ranges (N from 1 to 6000,
D any multiple of 8 (bf16) or 4 (fp32) up to 2048, V from 1 to 150000), so they
reach tile choices, chunk counts, ragged tails and vocabulary-split factors of
the backward that no hand-written case names. Each case is sized so that the
oracle finishes in about a second.
"""
import numpy as np
import pytest
import torch

import workloads
from parity import parity, parity_backward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _shapes(seed, count, budget):
    """count (N, D, V, dtype) with N*D*V <= budget: every other one drawn
    log-uniformly over the whole ranges, the others with N >= 512 and
    V >= 4000 (the sizes where the planner picks larger tiles and several
    chunks) and D log-uniform up to what the budget leaves."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        dt = "bf16" if rng.random() < 0.8 else "fp32"
        step = 8 if dt == "bf16" else 4
        if len(out) % 2 == 0:
            N = int(np.exp(rng.uniform(0, np.log(6000))))
            V = int(np.exp(rng.uniform(0, np.log(150000))))
            dmax = 2048
        else:
            N = int(np.exp(rng.uniform(np.log(512), np.log(6000))))
            V = int(np.exp(rng.uniform(np.log(4000), np.log(150000))))
            dmax = min(2048, int(budget // (N * V)))
        if dmax < step:
            continue
        D = step * int(np.exp(rng.uniform(0, np.log(dmax // step))))
        if N * D * V <= budget:
            out.append((N, D, V, dt))
    return out


FWD_SHAPES = _shapes(2024, 24, 1.5e10)
BWD_SHAPES = _shapes(4048, 12, 1.5e9)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401  (fails loudly if the library is missing)


def _inputs(N, D, V, dt, seed):
    std = 1.0 if dt == "bf16" else 0.5
    return workloads.make_custom(N, D, V, dt, seed=seed, device=DEV, h_std=std,
                                 w_std=2.0 / np.sqrt(D))


@pytest.mark.parametrize("N,D,V,dt", FWD_SHAPES, ids=lambda v: str(v))
def test_random_shape_forward(N, D, V, dt):
    print(f"[random fwd] N={N} D={D} V={V} {dt}", flush=True)
    H, W, y = _inputs(N, D, V, dt, seed=N + 3 * D + 7 * V)
    parity(H, W, y, what=f"random fwd N={N} D={D} V={V} {dt}")


@pytest.mark.parametrize("N,D,V,dt", BWD_SHAPES, ids=lambda v: str(v))
def test_random_shape_backward(N, D, V, dt):
    print(f"[random bwd] N={N} D={D} V={V} {dt}", flush=True)
    H, W, y = _inputs(N, D, V, dt, seed=5 * N + D + 11 * V)
    g = torch.linspace(0.25, 1.75, N, dtype=torch.float32).to(DEV)
    parity_backward(H, W, y, g, what=f"random bwd N={N} D={D} V={V} {dt}")


def _quant_shapes(seed, count, budget):
    """count (N, D, V, bits, group): 4 or 8 bits, groups of 8 to 256. Every
    other one has D a multiple of the group up to 4096 and N, V log-uniform;
    the others D from 2048 to 8192 and V from 20000 to 60000 with few rows, so
    that the head runs in several dequantisation slices (about 256 MB of bf16
    each). N*D*V <= budget."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        bits = int(rng.choice([4, 8]))
        group = int(rng.choice([8, 16, 32, 64, 128, 256]))
        if len(out) % 2 == 0:
            D = group * int(rng.integers(1, max(2, 4096 // group)))
            N = int(np.exp(rng.uniform(0, np.log(3000))))
            V = int(np.exp(rng.uniform(0, np.log(60000))))
        else:
            D = group * int(rng.integers(max(1, 2048 // group), 8192 // group + 1))
            V = int(rng.integers(20000, 60001))
            N = int(min(64, max(1, budget // (D * V))))
        if N * D * V <= budget:
            out.append((N, D, V, bits, group))
    return out


QUANT_SHAPES = _quant_shapes(606, 10, 3e9)


@pytest.mark.parametrize("N,D,V,bits,group", QUANT_SHAPES, ids=lambda v: str(v))
def test_random_shape_quant_head(N, D, V, bits, group):
    """The quantised head's forward and frozen-head backward against the
    oracle on the dequantised head (oracle.dequantize), every row."""
    import oracle
    import linear_cross_entropy_amd as flce
    from parity import check_bwd, check_close
    print(f"[random quant] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=N + V + D, device=DEV,
                                                       w_std=1.0 / np.sqrt(D))
    loss, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV)
    dH = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group)
    torch.cuda.synchronize()
    bits16 = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    Wq = torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).view(torch.bfloat16)
    rl, rs, _ = oracle.forward(H.cpu(), Wq, y.cpu())
    check_close(lse.cpu().numpy(), rs, torch.bfloat16, "random quant lse")
    check_close(loss.cpu().numpy(), rl, torch.bfloat16, "random quant loss")
    ref = oracle.backward(H.cpu(), Wq, y.cpu(), g.cpu(), want_dW=False)
    check_bwd(dH.cpu().numpy(), ref["dH"], ref["dH_abs"], torch.bfloat16, V, "random quant dH")
