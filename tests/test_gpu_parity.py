"""GPU parity: the HIP path against the float64 oracle on the same seeded bits.

Every case runs the library through its C ABI (via the ctypes binding) and
the oracle on the host. Large workloads compare a sampled subset of rows
(first, last and seeded random rows) against the oracle and check the bound
invariants max z <= lse <= max z + ln V (via loss >= 0 and finiteness) on
every row; every row of the large workloads is also compared with a plain
PyTorch fp32 computation on the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import BOUNDARY_SHAPES, EDGE, check_close, gpu_forward, parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401  (fails loudly if the library is missing)


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ benchmark workloads
@pytest.mark.parametrize("name,sample", [
    ("tiny_fp32", None),
    ("small_bf16", None),
    ("medium_bf16", 256),
    ("prod_bf16", 96),
    ("stress_bf16", 48),
])
def test_workload_parity(name, sample):
    """Every row where the oracle is cheap; otherwise a seeded sample plus the 32
    rows with the largest lse (largest logits, so the largest fp32 rounding)."""
    w = workloads.WORKLOADS[name]
    _log(f"[parity] {w.describe()} sample={sample}")
    H, W, y = workloads.make(w, DEV)
    rows = None
    if sample is not None:
        _, lse_gpu = gpu_forward(H, W, y)
        top = np.argsort(lse_gpu)[-32:]
        rows = np.union1d(workloads.subset_rows(w.N, sample).numpy(), top)
    loss, lse, err = parity(H, W, y, rows=rows, what=name)
    assert np.isfinite(loss).all() and np.isfinite(lse).all()
    assert (loss >= -2e-3).all(), "loss below 0 beyond rounding"
    _log(f"[parity] {name}: max |d| = {err:.3e}")


@pytest.mark.parametrize("name", ["medium_bf16", "prod_bf16", "stress_bf16"])
def test_every_row_against_torch_fp32(name):
    """Every row at the full size against a plain PyTorch computation on the
    GPU: the fp32 product of the bf16 inputs (exact products, fp32 sums), then
    logsumexp and the target logit per row. It shares nothing with the
    library or the oracle. The gate is the bf16 tolerance; both sides sum in
    fp32 in different orders, so the 16 rows where they differ most also go
    to the float64 oracle, which decides (at stress the outlier logits reach
    a few hundred and the two differ by up to ~1e-3 there)."""
    w = workloads.WORKLOADS[name]
    _log(f"[torch] {w.describe()} all rows")
    H, W, y = workloads.make(w, DEV)
    loss, lse = gpu_forward(H, W, y)
    Wt = W.float().t().contiguous()
    ref_lse, ref_loss = [], []
    for r0 in range(0, w.N, 1024):
        Z = torch.mm(H[r0:r0 + 1024].float(), Wt)
        l = torch.logsumexp(Z, dim=1)
        ref_lse.append(l.cpu())
        ref_loss.append((l - Z.gather(1, y[r0:r0 + 1024].long()[:, None])[:, 0]).cpu())
        del Z
    del Wt
    t_lse = torch.cat(ref_lse).double().numpy()
    t_loss = torch.cat(ref_loss).double().numpy()
    e1 = check_close(lse, t_lse, H.dtype, f"{name} lse vs torch")
    e2 = check_close(loss, t_loss, H.dtype, f"{name} loss vs torch")
    worst = np.argsort(np.maximum(np.abs(lse - t_lse), np.abs(loss - t_loss)))[-16:]
    rl, rs, _ = oracle.forward(H.cpu(), W.cpu(), y.cpu(), rows=worst)
    e3 = check_close(lse[worst], rs, H.dtype, f"{name} lse on the rows torch disagrees most")
    e4 = check_close(loss[worst], rl, H.dtype, f"{name} loss on the rows torch disagrees most")
    et = max(np.abs(t_lse[worst] - rs).max(), np.abs(t_loss[worst] - rl).max())
    _log(f"[torch] {name}: max |d| vs torch: lse {e1:.3e} loss {e2:.3e}; on those 16 rows vs the "
         f"oracle: kernel {max(e3, e4):.3e}, torch {et:.3e}")


# ------------------------------------------------------------------ edge grid
@pytest.mark.parametrize("N,D,V,dt", EDGE, ids=lambda v: str(v))
def test_edge_shapes(N, D, V, dt):
    std = 1.0 if dt == "bf16" else 0.5
    H, W, y = workloads.make_custom(N, D, V, dt, seed=N * 7 + V, device=DEV, h_std=std,
                                    w_std=0.5 / math.sqrt(D) * 4)
    _log(f"[edge] N={N} D={D} V={V} {dt}")
    parity(H, W, y, what=f"edge N={N} D={D} V={V} {dt}")


@pytest.mark.parametrize("N,D,V,dt", [(5, 1 << 21, 1000, "bf16"), (3, 1 << 20, 300, "fp32")],
                         ids=lambda v: str(v))
def test_longest_rows_one_tile_per_chunk(N, D, V, dt):
    """Rows of 4 MiB (D = 2^21 bf16, 2^20 fp32): one 256-row vocabulary tile
    of W is then 1 GiB, so the planner's limit of 2^31 bytes per chunk (one
    buffer resource) leaves one tile per chunk, and every tile runs 32768
    k-stages. Against the oracle on every row."""
    import linear_cross_entropy_amd as flce
    plan = flce.flce_get_plan(N, D, V, dt)
    assert plan["chunks"] == plan["vocab_tiles"] > 1, plan
    assert plan["tile_vocab"] * D * (2 if dt == "bf16" else 4) < 2 ** 31
    _log(f"[long] N={N} D={D} V={V} {dt} plan {plan}")
    H, W, y = workloads.make_custom(N, D, V, dt, seed=23, device=DEV, h_std=1.0,
                                    w_std=1.0 / math.sqrt(D))
    y[0] = V - 1                      # a target in the last, ragged tile
    _, _, err = parity(H, W, y, what=f"long rows N={N} D={D} V={V} {dt}")
    _log(f"[long] max |d| = {err:.3e}")


@pytest.mark.parametrize("N,D,V", BOUNDARY_SHAPES, ids=lambda v: str(v))
def test_targets_on_tile_and_chunk_boundaries(N, D, V):
    """Targets at 0, V-1 and either side of every tile and chunk boundary."""
    import linear_cross_entropy_amd as flce
    plan = flce.flce_get_plan(N, D, V, "bf16")
    BV, T, C = plan["tile_vocab"], plan["vocab_tiles"], plan["chunks"]
    base, rem = divmod(T, C)
    marks = {0, V - 1}
    for t in range(1, T):
        marks.update({t * BV - 1, t * BV})
    for c in range(1, C):
        s = (c * base + min(c, rem)) * BV
        marks.update({s - 1, s})
    # every row position inside the first MFMA tiles (16x16: 4 lane groups x
    # 4 registers; 32x32: 2 x 16), both 32-row blocks' edges, and the edge
    # between the two waves that split a tile's vocabulary
    marks.update(range(0, 48))
    for sub in (63, 64, 127, 128, BV // 2 - 1, BV // 2, BV // 2 + 15, BV // 2 + 16):
        marks.add(sub)
    marks = sorted(m for m in marks if 0 <= m < V)
    H, W, _ = workloads.make_custom(N, D, V, "bf16", seed=11, device=DEV)
    y = torch.tensor([marks[i % len(marks)] for i in range(N)], dtype=torch.int32, device=DEV)
    _log(f"[boundary] N={N} D={D} V={V} tile={BV} chunks={C}")
    parity(H, W, y, what=f"boundary targets N={N} D={D} V={V}")


def test_out_of_range_targets_give_nan_loss():
    N, D, V = 64, 128, 1000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=3, device=DEV)
    y[0] = -1
    y[1] = V
    y[2] = V + 200          # inside the padded part of the last tile
    y[3] = 2**31 - 1
    loss, lse = gpu_forward(H, W, y)
    assert np.isnan(loss[:4]).all()
    assert np.isfinite(lse).all() and np.isfinite(loss[4:]).all()
    parity(H, W, y, what="out-of-range targets")


def test_large_logit_held_over_many_tiles():
    """A logit near 1000 in the first tile of every vocabulary chunk, then ~100
    tiles whose maximum stays below it, so each of those tiles must rescale the
    running sum by exactly 1. (A rescale that re-derives the base-2 offset with
    an extra rounding drifts by up to 6e-5 per tile at this magnitude, several
    1e-3 in lse over a chunk.)"""
    import linear_cross_entropy_amd as flce
    N, D, V = 8192, 64, 262144
    plan = flce.flce_get_plan(N, D, V, "bf16")
    T, C, BV = plan["vocab_tiles"], plan["chunks"], plan["tile_vocab"]
    assert T // C >= 64, "the shape must give long chunks"
    base, rem = divmod(T, C)
    starts = [(c * base + min(c, rem)) * BV for c in range(C)]
    g = torch.Generator().manual_seed(17)
    H = torch.randn(N, D, generator=g)
    H[:, 0] = 1000.0 + 8.0 * (torch.arange(N) % 16)      # exact in bf16 (spacing 8 at 1000)
    W = torch.randn(V, D, generator=g) * 0.3
    W[:, 0] = 0.0
    W[starts, 0] = 1.0                                    # the first row of every chunk carries the large logit
    H, W = H.to(torch.bfloat16).to(DEV), W.to(torch.bfloat16).to(DEV)
    y = torch.randint(0, V, (N,), generator=g, dtype=torch.int32).to(DEV)
    rows = workloads.subset_rows(N, 256, seed=5).numpy()
    _, lse, err = parity(H, W, y, rows=rows, what="large logit over many tiles")
    assert (lse > 990.0).all()
    _log(f"[parity] large logit over many tiles: max |d| = {err:.3e}")


def test_zero_weights_give_log_V():
    """W = 0: every logit is 0, lse = loss = ln V. Padded vocabulary rows must not count."""
    for V in (1, 7, 255, 257, 50257):
        N, D = 65, 64
        H = torch.randn(N, D, device=DEV).to(torch.bfloat16)
        W = torch.zeros(V, D, dtype=torch.bfloat16, device=DEV)
        y = torch.randint(0, V, (N,), device=DEV, dtype=torch.int32)
        loss, lse = gpu_forward(H, W, y)
        check_close(lse, np.full(N, math.log(V)), torch.float32, f"W=0 lse V={V}")
        check_close(loss, np.full(N, math.log(V)), torch.float32, f"W=0 loss V={V}")


def test_shift_invariance_large_offset():
    """H'=[H, c], W'=[W, 1]: lse' = lse + c, loss' = loss; c=1024 overflows a non-stable exp."""
    from oracle_pins import augment_shift
    N, D, V = 128, 256, 3000
    for dt, c in (("bf16", 1024.0), ("fp32", 64.0)):
        H, W, y = workloads.make_custom(N, D, V, dt, seed=5, device=DEV)
        Hp, Wp = augment_shift(H, W, c)
        _, lse0, _ = parity(H, W, y, what=f"unshifted {dt}")
        loss1, lse1, _ = parity(Hp, Wp, y, what=f"shifted {dt} c={c}")
        check_close(lse1 - c, lse0.astype(np.float64), Hp.dtype, "lse' - c vs lse")


def test_permuted_vocabulary():
    """Permuting W's rows and remapping targets leaves loss and lse unchanged."""
    N, D, V = 256, 512, 9000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=9, device=DEV)
    g = torch.Generator().manual_seed(9)
    perm = torch.randperm(V, generator=g)
    inv = torch.argsort(perm)
    l0, s0 = gpu_forward(H, W, y)
    l1, s1 = gpu_forward(H, W[perm.to(DEV)].contiguous(), inv.to(DEV)[y.long()].to(torch.int32))
    check_close(l1, l0.astype(np.float64), torch.bfloat16, "permuted loss")
    check_close(s1, s0.astype(np.float64), torch.bfloat16, "permuted lse")


def test_rows_are_independent():
    """A row's loss and lse do not depend on the other rows of the batch: a
    prefix and a slice from the middle, run as batches of their own (other row
    blocks, other chunk splits), agree with the full batch's rows."""
    N, D, V = 1100, 512, 20000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=12, device=DEV)
    l0, s0 = gpu_forward(H, W, y)
    for a, b in ((0, 300), (517, 889)):
        l1, s1 = gpu_forward(H[a:b].contiguous(), W, y[a:b].contiguous())
        check_close(l1, l0[a:b].astype(np.float64), torch.bfloat16, f"rows [{a}, {b}) loss")
        check_close(s1, s0[a:b].astype(np.float64), torch.bfloat16, f"rows [{a}, {b}) lse")


def test_nan_input_propagates_to_its_row_only():
    N, D, V = 16, 64, 700
    H, W, y = workloads.make_custom(N, D, V, "fp32", seed=2, device=DEV)
    H[5, 7] = float("nan")
    loss, lse = gpu_forward(H, W, y)
    assert np.isnan(loss[5]) and np.isnan(lse[5])
    keep = np.arange(N) != 5
    assert np.isfinite(loss[keep]).all() and np.isfinite(lse[keep]).all()


# ------------------------------------------------------------------ properties
def test_deterministic_bits():
    H, W, y = workloads.make_custom(700, 1024, 40000, "bf16", seed=4, device=DEV)
    a = gpu_forward(H, W, y)
    b = gpu_forward(H, W, y)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_outputs_fully_overwritten_and_guards_untouched():
    """NaN-poisoned outputs are fully overwritten; canaries around outputs and
    the caller workspace stay intact; lse may be omitted."""
    import linear_cross_entropy_amd as flce
    N, D, V = 300, 256, 5000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=6, device=DEV)
    pad = 64
    out = torch.full((N + 2 * pad,), float("nan"), device=DEV)
    lse = torch.full((N + 2 * pad,), float("nan"), device=DEV)
    out[:pad] = 7.0
    out[-pad:] = 7.0
    nbytes = flce.flce_workspace_bytes(N, D, V, "bf16")
    ws = torch.full((nbytes + 2 * 256,), 0xA5, dtype=torch.uint8, device=DEV)
    ws_in = ws[256:256 + nbytes]
    flce.flce_forward_ws(H, W, y, ws_in, loss=out[pad:pad + N], lse=lse[pad:pad + N])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o[pad:pad + N]).all()
    assert (o[:pad] == 7.0).all() and (o[-pad:] == 7.0).all()
    assert np.isnan(lse.cpu().numpy()[:pad]).all()
    wsc = ws.cpu().numpy()
    assert (wsc[:256] == 0xA5).all() and (wsc[256 + nbytes:] == 0xA5).all()
    rl, rs, _ = oracle.forward(H.cpu(), W.cpu(), y.cpu())
    check_close(o[pad:pad + N], rl, torch.bfloat16, "ws loss")
    check_close(lse.cpu().numpy()[pad:pad + N], rs, torch.bfloat16, "ws lse")
    # loss only
    loss_only, none = flce.flce_forward(H, W, y, want_lse=False)
    torch.cuda.synchronize()
    assert none is None
    check_close(loss_only.cpu().numpy(), rl, torch.bfloat16, "loss only")


def test_partials_then_merge_equals_forward():
    import linear_cross_entropy_amd as flce
    N, D, V = 513, 512, 20000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=8, device=DEV)
    ws = flce.workspace(N, D, V, "bf16", DEV)
    flce.flce_partials(H, W, y, ws)
    l1, s1 = flce.flce_merge(y, D, V, "bf16", ws)
    l0, s0 = flce.flce_forward_ws(H, W, y, ws)
    torch.cuda.synchronize()
    assert torch.equal(l0, l1) and torch.equal(s0, s1)


def test_no_logits_sized_allocation_at_production_shape():
    """Device memory grows by the workspace only, far below one N x V fp32 matrix."""
    import linear_cross_entropy_amd as flce
    w = workloads.WORKLOADS["prod_bf16"]
    H, W, y = workloads.make(w, DEV)
    loss = torch.empty(w.N, device=DEV)
    lse = torch.empty(w.N, device=DEV)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    flce.flce_forward(H, W, y, loss=loss, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    ws = flce.flce_workspace_bytes(w.N, w.D, w.V, "bf16")
    assert ws < 0.01 * w.N * w.V * 4
    # the stream-ordered pool may keep the freed workspace: at most the workspace
    # (rounded to the pool's granularity) may be missing afterwards
    assert free0 - free1 <= ws + (64 << 20)
