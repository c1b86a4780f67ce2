"""The quantised-head forward (flce_forward_quant) on the GPU.

The dequantised bf16 weights the library leaves in its workspace must equal
oracle.dequantize bit for bit; a vocabulary that fits one slice must give the
same bits as flce_forward on those weights; and several slices must match
the oracle (dequantize, then the float64 forward) on every row, with targets
on every slice boundary.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401  (fails loudly if the library is missing)


def _as_bf16(bits16):
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("bits,group,D", [(8, 64, 256), (4, 32, 256), (4, 256, 256),
                                          (8, 8, 264), (4, 16, 272)])
def test_single_slice_dequant_bits_and_dense_equality(bits, group, D):
    """Several bit widths and group sizes, including D = 264 and 272 (groups of 8
    and 16: 33 and 17 groups a row)."""
    import linear_cross_entropy_amd as flce
    N, V = 300, 5003
    print(f"[quant] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=bits + group, device=DEV)
    # a few rows where two float32 roundings and a fused multiply-add differ
    third = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(3.0, dtype=torch.float32)
    scales[:3] = third.item()
    biases[:3] = -1.0
    if bits == 8:
        codes[:3] = 3
    else:
        codes[:3] = 0x33
    nbytes = flce.flce_forward_quant_workspace_bytes(N, D, V, bits, group)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    loss, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group, workspace=ws)
    torch.cuda.synchronize()
    ref_bits = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    got_bits = ws[:V * D * 2].cpu().numpy().view(np.uint16).reshape(V, D)
    bad = np.nonzero(got_bits != ref_bits)
    assert bad[0].size == 0, f"dequantised weight ({bad[0][0]}, {bad[1][0]}) differs from the oracle"
    assert np.all(ref_bits[:3] == 0)                     # the rows above: exactly 0, not 2.98e-8
    W = _as_bf16(ref_bits).to(DEV)
    loss_d, lse_d = flce.flce_forward(H, W, y)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss_d) and torch.equal(lse, lse_d)
    rl, rs, _ = oracle.forward(H.cpu(), _as_bf16(ref_bits), y.cpu())
    check_close(lse.cpu().numpy(), rs, torch.bfloat16, "quant lse")
    check_close(loss.cpu().numpy(), rl, torch.bfloat16, "quant loss")


@pytest.mark.parametrize("bits,group", [(8, 128), (4, 64)])
def test_several_slices_against_the_oracle(bits, group):
    """D = 16384 gives 6144-row slices: V = 13000 runs as 6144 + 6144 + 712,
    with targets on both sides of every slice boundary and one ignored row."""
    import linear_cross_entropy_amd as flce
    N, D, V = 64, 16384, 13000
    print(f"[quant] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=97 + bits, device=DEV,
                                                       w_std=1.0 / np.sqrt(D))
    marks = [0, 6143, 6144, 6145, 12287, 12288, 12999, -1]
    y[:len(marks)] = torch.tensor(marks, dtype=torch.int32, device=DEV)
    loss, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    loss2, lse2 = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    torch.cuda.synchronize()
    same = torch.equal(loss.view(torch.int32), loss2.view(torch.int32)) and \
        torch.equal(lse.view(torch.int32), lse2.view(torch.int32))   # bit patterns: the ignored row is NaN
    assert same, "second call differs"
    ref_bits = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    rl, rs, _ = oracle.forward(H.cpu(), _as_bf16(ref_bits), y.cpu())
    e1 = check_close(lse.cpu().numpy(), rs, torch.bfloat16, "quant slices lse")
    e2 = check_close(loss.cpu().numpy(), rl, torch.bfloat16, "quant slices loss")
    assert np.isnan(loss[len(marks) - 1].item())
    print(f"[quant] max |d| lse {e1:.3e} loss {e2:.3e}", flush=True)


def test_binding_rejects_bad_formats():
    import linear_cross_entropy_amd as flce
    H, codes, scales, biases, y = workloads.make_quant(8, 64, 100, 8, 32, seed=3, device=DEV)
    with pytest.raises(ValueError):
        flce.flce_forward_quant(H, codes, scales, biases, y, 3, 32)
    with pytest.raises(ValueError):
        flce.flce_forward_quant(H, codes, scales, biases, y, 8, 24)
    with pytest.raises(ValueError):
        flce.flce_forward_quant(H, codes[:, :32].contiguous(), scales, biases, y, 8, 32)


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32)])
def test_backward_single_slice_equals_the_dense_backward(bits, group):
    """dH for a vocabulary that fits one slice: the same bits as flce_backward's
    dH on the dequantised bf16 head, and the oracle's dH within the backward
    bound."""
    import linear_cross_entropy_amd as flce
    from parity import check_bwd
    N, D, V = 300, 256, 5003
    print(f"[quant bwd] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=11 + bits, device=DEV)
    g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV)
    _, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    dH = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group)
    torch.cuda.synchronize()
    ref_bits = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    W = _as_bf16(ref_bits).to(DEV)
    dH_d, _ = flce.flce_backward(H, W, y, lse, g)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH_d)
    ref = oracle.backward(H.cpu(), _as_bf16(ref_bits), y.cpu(), g.cpu(), want_dW=False)
    check_bwd(dH.cpu().numpy(), ref["dH"], ref["dH_abs"], torch.bfloat16, V, "quant bwd dH")


@pytest.mark.parametrize("bits,group", [(8, 128), (4, 64)])
def test_backward_several_slices_against_the_oracle(bits, group):
    """Three vocabulary slices (D = 16384, V = 13000), each dH product further
    split over its vocabulary (64 rows leave CUs idle): nine partial products
    added in order. Targets on the slice boundaries and one outside [0, V)."""
    import linear_cross_entropy_amd as flce
    from parity import check_bwd
    N, D, V = 64, 16384, 13000
    print(f"[quant bwd] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=31 + bits, device=DEV,
                                                       w_std=1.0 / np.sqrt(D))
    marks = [0, 6143, 6144, 12287, 12288, 12999, -1]
    y[:len(marks)] = torch.tensor(marks, dtype=torch.int32, device=DEV)
    g = torch.linspace(0.25, 1.75, N, dtype=torch.float32, device=DEV)
    _, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    dH = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group)
    dH2 = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH2), "second call differs"
    ref_bits = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    ref = oracle.backward(H.cpu(), _as_bf16(ref_bits), y.cpu(), g.cpu(), want_dW=False)
    e, rel = check_bwd(dH.cpu().numpy(), ref["dH"], ref["dH_abs"], torch.bfloat16, V, "quant slices bwd dH")
    print(f"[quant bwd] max |d| {e:.3e}, relative Frobenius error {rel:.2e}", flush=True)


def test_autograd_quant_head():
    import linear_cross_entropy_amd as flce
    N, D, V = 200, 128, 3001
    H0, codes, scales, biases, y = workloads.make_quant(N, D, V, 4, 32, seed=71, device=DEV)
    weights = torch.linspace(-1.0, 2.0, N, dtype=torch.float32, device=DEV)
    H = H0.clone().requires_grad_(True)
    loss = flce.linear_cross_entropy_quant(H, codes, scales, biases, y, 4, 32)
    (loss * weights).sum().backward()
    torch.cuda.synchronize()
    loss_d, lse_d = flce.flce_forward_quant(H0, codes, scales, biases, y, 4, 32)
    dH_d = flce.flce_backward_quant(H0, codes, scales, biases, y, lse_d, weights.contiguous(), 4, 32)
    torch.cuda.synchronize()
    assert torch.equal(loss.detach(), loss_d)
    assert H.grad.dtype == torch.bfloat16 and torch.equal(H.grad, dH_d.to(torch.bfloat16))


@pytest.mark.parametrize("N,D,V,bits,group", [
    (1, 8, 1, 4, 8),            # one token, one vocabulary row, the smallest D and group
    (3, 16, 17, 8, 8),
    (257, 1024, 3073, 4, 128),  # ragged rows and vocabulary, one slice
    (5, 65536, 6500, 8, 64),    # 3072-row slices (the minimum) and a ragged last one
], ids=lambda v: str(v))
def test_degenerate_and_ragged_quant_shapes(N, D, V, bits, group):
    import linear_cross_entropy_amd as flce
    from parity import check_bwd
    print(f"[quant edge] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=N + V, device=DEV,
                                                       w_std=1.0 / np.sqrt(D))
    y[0] = V - 1
    loss, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group)
    g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV)
    dH = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group)
    torch.cuda.synchronize()
    ref_bits = oracle.dequantize(codes.cpu(), scales.cpu(), biases.cpu(), bits, group)
    Wq = _as_bf16(ref_bits)
    rl, rs, _ = oracle.forward(H.cpu(), Wq, y.cpu())
    check_close(lse.cpu().numpy(), rs, torch.bfloat16, "quant edge lse")
    check_close(loss.cpu().numpy(), rl, torch.bfloat16, "quant edge loss")
    ref = oracle.backward(H.cpu(), Wq, y.cpu(), g.cpu(), want_dW=False)
    check_bwd(dH.cpu().numpy(), ref["dH"], ref["dH_abs"], torch.bfloat16, V, "quant edge dH")
