"""Pins for the oracle: checks that tie it to the mathematics, not to itself.

Each pin takes ``fwd(H, W, y, rows=None) -> (loss, lse, z_target)`` (float64
numpy arrays) and raises AssertionError when the implementation disagrees with
a closed form, an invariant, an exact brute force, or a hand-worked example.
The definition pinned is the one on the page "Een gefuseerde forward-kernel
voor lineaire cross-entropy op Apple-GPU's" (section 1): Z = H W^T,
loss_i = logsumexp(Z_i) - Z_{i, y_i}.

The same pins run against deliberately broken copies of the oracle in
``test_oracle_mutants.py``; every broken copy must fail at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f32(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32))


def _y(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32))


def _close(a, b, tol, what, scale=None):
    """|a - b| <= tol * max(1, |scale|) elementwise (scale defaults to b)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    ref = np.abs(b) if scale is None else np.abs(np.asarray(scale, dtype=np.float64))
    bound = tol * np.maximum(1.0, ref)
    if not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: got {a.flat[i]!r}, want {b.flat[i]!r} (|d|={err.flat[i]:.3e})")


# ---------------------------------------------------------------- exact brute force
def exact_reference(H: torch.Tensor, W: torch.Tensor, y: torch.Tensor, digits: int = 50):
    """Logits in exact rational arithmetic, then exp and ln in 50-digit decimal.

    The inputs are bf16 or fp32 numbers, i.e. dyadic rationals, so every
    logit is exact. The log-sum-exp is evaluated as ln of the sum of e^(z_v),
    with the sum factored at the largest logit only to keep the decimal
    exponent range small. Returns (loss, lse) as Decimal lists.
    """
    getcontext().prec = digits
    h = H.to(torch.float32).tolist()
    w = W.to(torch.float32).tolist()
    out_loss, out_lse = [], []
    for i, hrow in enumerate(h):
        z = [sum((Fraction(a) * Fraction(b) for a, b in zip(hrow, wrow)), Fraction(0)) for wrow in w]
        zd = [Decimal(q.numerator) / Decimal(q.denominator) for q in z]
        top = max(zd)
        total = sum(((v - top).exp() for v in zd), Decimal(0))
        lse = top + total.ln()
        t = int(y[i])
        out_lse.append(lse)
        out_loss.append(lse - zd[t] if 0 <= t < len(w) else Decimal("NaN"))
    return out_loss, out_lse


def pin_exact_bruteforce(fwd):
    """Tiny random problems against the exact reference (|d| <= 1e-13)."""
    rng = np.random.default_rng(20260719)
    for case in range(10):
        N = int(rng.integers(1, 5))
        D = int(rng.integers(1, 17))
        V = int(rng.integers(1, 41))
        scale = float(rng.choice([0.1, 1.0, 4.0]))
        Hn = rng.standard_normal((N, D)).astype(np.float32) * scale
        Wn = rng.standard_normal((V, D)).astype(np.float32) * scale
        mk = _bf16 if case % 2 == 0 else _f32
        H, W = mk(Hn), mk(Wn)
        y = _y(rng.integers(0, V, N))
        loss, lse, _ = fwd(H, W, y)
        rl, rs = exact_reference(H, W, y)
        _close(lse, [float(v) for v in rs], 1e-13, f"exact lse case {case}")
        _close(loss, [float(v) for v in rl], 1e-13, f"exact loss case {case}")


def pin_hand_examples(fwd):
    """Hand-worked closed forms stored in tests/golden/hand_examples.json."""
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        data = json.load(f)
    getcontext().prec = 50
    env = {"ln": lambda x: Decimal(x).ln(), "exp": lambda x: Decimal(x).exp(), "__builtins__": {}}

    def ev(expr):
        # numbers in the expressions become Decimals before evaluation
        import re
        return eval(re.sub(r"(\d+(?:\.\d+)?)", r"Decimal('\1')", expr), {**env, "Decimal": Decimal})

    for ex in data["examples"]:
        for mk in (_bf16, _f32):
            loss, lse, _ = fwd(mk(ex["H"]), mk(ex["W"]), _y(ex["y"]))
            _close(lse, [float(ev(e)) for e in ex["lse"]], 1e-15, f"{ex['name']} lse")
            _close(loss, [float(ev(e)) for e in ex["loss"]], 1e-15, f"{ex['name']} loss")


# ---------------------------------------------------------------- closed forms
def pin_zero_weights(fwd):
    """W = 0 (or H = 0) makes every logit 0, so lse = loss = ln V exactly."""
    rng = np.random.default_rng(1)
    for V in (1, 2, 3, 31, 256, 257, 1000):
        D = 8
        H = _bf16(rng.standard_normal((3, D)))
        W = _bf16(np.zeros((V, D)))
        y = _y(rng.integers(0, V, 3))
        loss, lse, _ = fwd(H, W, y)
        _close(lse, np.full(3, math.log(V)), 1e-15, f"W=0 lse V={V}")
        _close(loss, np.full(3, math.log(V)), 1e-15, f"W=0 loss V={V}")
        loss, lse, _ = fwd(_f32(np.zeros((3, D))), _f32(rng.standard_normal((V, D))), y)
        _close(loss, np.full(3, math.log(V)), 1e-15, f"H=0 loss V={V}")


def pin_single_word(fwd):
    """V = 1: the only logit is the target, loss = 0 exactly; lse = z_0."""
    H = _f32([[1.5, -2.0, 0.25], [3.0, 0.0, 1.0]])
    W = _f32([[2.0, 1.0, -4.0]])
    loss, lse, _ = fwd(H, W, _y([0, 0]))
    _close(loss, [0.0, 0.0], 0.0, "V=1 loss")
    _close(lse, [3.0 - 2.0 - 1.0, 6.0 - 4.0], 0.0, "V=1 lse")


def pin_two_words(fwd):
    """V = 2 with W = I: z = h, loss = ln(1 + e^(z_other - z_y))."""
    rows = [[0.5, -1.25], [8.0, 8.0], [-3.0, 20.0], [100.0, -100.0]]
    H = _f32(rows)
    W = _f32([[1.0, 0.0], [0.0, 1.0]])
    for t in (0, 1):
        loss, lse, zt = fwd(H, W, _y([t] * len(rows)))
        want = [math.log1p(math.exp(r[1 - t] - r[t])) for r in rows]
        # loss = lse - z_y cancels: its rounding is relative to |lse|, not to the loss
        _close(loss, want, 1e-15, f"V=2 loss y={t}", scale=[max(map(abs, r)) for r in rows])
        _close(zt, [r[t] for r in rows], 0.0, f"V=2 target logit y={t}")
        _close(lse, [max(r) + math.log1p(math.exp(min(r) - max(r))) for r in rows], 1e-15, "V=2 lse")


def pin_equal_logits(fwd):
    """All W rows equal: every logit equals z, so lse = z + ln V, loss = ln V."""
    rng = np.random.default_rng(2)
    D, V = 5, 77
    h = np.array([[1.0, 2.0, -1.0, 0.5, 0.0]], np.float32)
    w = np.tile(np.array([[0.5, 0.25, 1.0, -2.0, 3.0]], np.float32), (V, 1))
    z = 0.5 + 0.5 - 1.0 - 1.0 + 0.0
    loss, lse, _ = fwd(_f32(h), _f32(w), _y([int(rng.integers(0, V))]))
    _close(lse, [z + math.log(V)], 1e-15, "equal logits lse")
    _close(loss, [math.log(V)], 1e-15, "equal logits loss")


# ---------------------------------------------------------------- invariants
def augment_shift(H: torch.Tensor, W: torch.Tensor, c: float, pad: int = 8):
    """H' = [H, c, 0...], W' = [W, 1, 0...]: every logit of every row grows by c."""
    N, D = H.shape
    V = W.shape[0]
    Hp = torch.zeros(N, D + pad, dtype=H.dtype, device=H.device)
    Wp = torch.zeros(V, D + pad, dtype=W.dtype, device=W.device)
    Hp[:, :D] = H
    Hp[:, D] = c
    Wp[:, :D] = W
    Wp[:, D] = 1.0
    return Hp, Wp


def pin_shift_invariance(fwd):
    """Adding c to a row's logits adds c to lse and leaves the loss unchanged."""
    rng = np.random.default_rng(3)
    N, D, V = 4, 24, 300
    for mk in (_bf16, _f32):
        H = mk(rng.standard_normal((N, D)))
        W = mk(rng.standard_normal((V, D)) * 0.5)
        y = _y(rng.integers(0, V, N))
        loss, lse, _ = fwd(H, W, y)
        for c in (1024.0, -1024.0, 64.0):
            Hp, Wp = augment_shift(H, W, c)
            loss2, lse2, _ = fwd(Hp, Wp, y)
            _close(lse2 - c, lse, 1e-12 * abs(c), f"shift lse c={c}")
            _close(loss2, loss, 1e-12 * abs(c), f"shift loss c={c}")


def pin_permutation(fwd):
    """Permuting W's rows and remapping the targets leaves loss and lse unchanged."""
    rng = np.random.default_rng(4)
    N, D, V = 6, 16, 97
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)))
    y = rng.integers(0, V, N)
    perm = rng.permutation(V)             # new row j holds old row perm[j]
    inv = np.argsort(perm)
    loss, lse, zt = fwd(H, W, _y(y))
    loss2, lse2, zt2 = fwd(H, W[torch.as_tensor(perm)], _y(inv[y]))
    _close(lse2, lse, 1e-14, "permuted lse")
    _close(loss2, loss, 1e-14, "permuted loss")
    _close(zt2, zt, 0.0, "permuted target logit")


def pin_row_independence(fwd):
    """A row's result does not depend on which other rows are computed."""
    rng = np.random.default_rng(5)
    N, D, V = 9, 12, 50
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)))
    y = _y(rng.integers(0, V, N))
    loss, lse, _ = fwd(H, W, y)
    rows = [7, 0, 3]
    loss2, lse2, _ = fwd(H, W, y, rows=rows)
    _close(loss2, loss[rows], 0.0, "row subset loss")
    _close(lse2, lse[rows], 0.0, "row subset lse")
    # and the result for a row is the result of that row alone
    for i in (0, 4, 8):
        l1, s1, _ = fwd(H[i:i + 1], W, y[i:i + 1])
        _close(l1, loss[i:i + 1], 0.0, f"row {i} alone")


def pin_bounds(fwd):
    """max z <= lse <= max z + ln V, and z_y <= lse, so loss >= 0."""
    rng = np.random.default_rng(6)
    N, D, V = 8, 32, 500
    H = _bf16(rng.standard_normal((N, D)) * 3)
    W = _bf16(rng.standard_normal((V, D)))
    y = _y(rng.integers(0, V, N))
    loss, lse, zt = fwd(H, W, y)
    z = H.double() @ W.double().T                  # the logits, used only for their max
    zmax = z.max(dim=1).values.numpy()
    assert np.all(lse >= zmax - 1e-12 * np.abs(zmax)), "lse below max logit"
    assert np.all(lse <= zmax + math.log(V) + 1e-12 * np.abs(zmax)), "lse above max + ln V"
    assert np.all(loss >= -1e-12), "negative loss"
    _close(zt, z[torch.arange(N), y.long()].numpy(), 1e-14, "target logit")


def pin_out_of_range_target(fwd):
    """A target outside [0, V) gives loss NaN; lse is unaffected."""
    rng = np.random.default_rng(7)
    N, D, V = 4, 8, 20
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)))
    good = _y([0, 5, 19, 3])
    bad = _y([-1, 5, 20, 2**31 - 1])
    l1, s1, _ = fwd(H, W, good)
    l2, s2, _ = fwd(H, W, bad)
    _close(s2, s1, 0.0, "lse with bad targets")
    assert np.isnan(l2[0]) and np.isnan(l2[2]) and np.isnan(l2[3]), "bad target not NaN"
    _close(l2[1:2], l1[1:2], 0.0, "good row next to bad rows")


def pin_nan_propagates(fwd):
    """A NaN in a row of H makes that row's lse and loss NaN, and only that row."""
    rng = np.random.default_rng(8)
    N, D, V = 3, 8, 30
    h = rng.standard_normal((N, D)).astype(np.float32)
    h[1, 3] = np.nan
    H = _f32(h)
    W = _f32(rng.standard_normal((V, D)))
    y = _y([1, 2, 3])
    loss, lse, _ = fwd(H, W, y)
    assert np.isnan(loss[1]) and np.isnan(lse[1])
    assert np.isfinite(loss[[0, 2]]).all() and np.isfinite(lse[[0, 2]]).all()


ALL_PINS = [
    pin_exact_bruteforce,
    pin_hand_examples,
    pin_zero_weights,
    pin_single_word,
    pin_two_words,
    pin_equal_logits,
    pin_shift_invariance,
    pin_permutation,
    pin_row_independence,
    pin_bounds,
    pin_out_of_range_target,
    pin_nan_propagates,
]


# ---------------------------------------------------------------- backward pins
# Each takes (fwd, bwd) with bwd(H, W, y, g, rows=None, want_dW=True) -> dict of
# float64 arrays dH, dH_abs (rows), dW, dW_abs (all rows). The backward is the
# gradient of sum_i g_i loss_i for the section 1 definition; the forward it is
# checked against is already pinned above.

def _richardson(f, x0: np.ndarray, idx, h: float) -> float:
    """d f / d x[idx] by central differences at steps h and h/2, combined to
    cancel the h^2 term. The steps are powers of two, so x +- h is exact in fp32
    for the |x| used here."""
    def central(step):
        xp = x0.copy()
        xm = x0.copy()
        xp[idx] += np.float32(step)
        xm[idx] -= np.float32(step)
        return (f(xp) - f(xm)) / (2.0 * step)
    return (4.0 * central(h / 2) - central(h)) / 3.0


def pin_bwd_finite_differences(fwd, bwd):
    """dH and dW against Richardson-extrapolated central differences of
    sum_i g_i loss_i, evaluated with the forward oracle (fp32 inputs)."""
    rng = np.random.default_rng(40)
    for case, (N, D, V) in enumerate([(3, 5, 7), (2, 3, 1), (4, 2, 11)]):
        Hn = (rng.standard_normal((N, D)) * 0.7).astype(np.float32)
        Wn = (rng.standard_normal((V, D)) * 0.7).astype(np.float32)
        y = _y(rng.integers(0, V, N))
        g = rng.uniform(0.5, 1.5, N).astype(np.float32)

        def F_of_H(h):
            loss, _, _ = fwd(_f32(h), _f32(Wn), y)
            return float(np.dot(g.astype(np.float64), loss))

        def F_of_W(w):
            loss, _, _ = fwd(_f32(Hn), _f32(w), y)
            return float(np.dot(g.astype(np.float64), loss))

        out = bwd(_f32(Hn), _f32(Wn), y, g)
        fd_H = np.array([[_richardson(F_of_H, Hn, (i, d), 2.0 ** -6) for d in range(D)] for i in range(N)])
        fd_W = np.array([[_richardson(F_of_W, Wn, (v, d), 2.0 ** -6) for d in range(D)] for v in range(V)])
        _close(out["dH"], fd_H, 2e-6, f"dH vs finite differences case {case}")
        _close(out["dW"], fd_W, 2e-6, f"dW vs finite differences case {case}")


def pin_bwd_zero_weights(fwd, bwd):
    """W = 0: every row's softmax is uniform, so dH = sum_v dZ_iv W_v = 0 and
    dW_v = sum_i g_i (1/V - [v == y_i]) H_i; the sizes of dW's terms are
    |g_i| (1/V + [v == y_i]) |H_i|."""
    rng = np.random.default_rng(41)
    N, D, V = 5, 6, 9
    Hn = rng.standard_normal((N, D)).astype(np.float32)
    yn = rng.integers(0, V, N)
    g = rng.uniform(-1, 1, N).astype(np.float32)
    out = bwd(_f32(Hn), _f32(np.zeros((V, D))), _y(yn), g)
    _close(out["dH"], np.zeros((N, D)), 0.0, "W=0 dH")
    want = np.zeros((V, D))
    want_abs = np.zeros((V, D))
    for i in range(N):
        for v in range(V):
            hit = 1.0 if v == yn[i] else 0.0
            want[v] += float(g[i]) * ((1.0 / V) - hit) * Hn[i].astype(np.float64)
            want_abs[v] += abs(float(g[i])) * ((1.0 / V) + hit) * np.abs(Hn[i].astype(np.float64))
    _close(out["dW"], want, 1e-14, "W=0 dW")
    # the sizes of the terms: |g_i| (1/V + [v == y_i]) |H_id| summed over i; dH's are all 0
    _close(out["dW_abs"], want_abs, 1e-14, "W=0 dW_abs")
    _close(out["dH_abs"], np.zeros((N, D)), 0.0, "W=0 dH_abs")


def pin_bwd_single_word(fwd, bwd):
    """V = 1: softmax is 1 and so is the one-hot, so both gradients vanish."""
    rng = np.random.default_rng(42)
    H = _bf16(rng.standard_normal((3, 8)))
    W = _bf16(rng.standard_normal((1, 8)))
    out = bwd(H, W, _y([0, 0, 0]), np.ones(3, np.float32))
    _close(out["dH"], np.zeros((3, 8)), 0.0, "V=1 dH")
    _close(out["dW"], np.zeros((1, 8)), 0.0, "V=1 dW")


def pin_bwd_identities(fwd, bwd):
    """sum_v dZ_iv = 0 for a valid target, so sum_v dW_v = 0; and
    <dH, H> = <dW, W> = sum_iv dZ_iv z_iv; each output is bounded by the sum
    of the absolute values of its terms."""
    rng = np.random.default_rng(43)
    N, D, V = 6, 16, 50
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)) * 0.5)
    y = _y(rng.integers(0, V, N))
    g = rng.uniform(0.1, 2.0, N).astype(np.float32)
    out = bwd(H, W, y, g)
    colsum = out["dW"].sum(axis=0)
    scale = out["dW_abs"].sum(axis=0)
    assert np.all(np.abs(colsum) <= 1e-12 * scale), "sum over the vocabulary of dW is not 0"
    lhs = float((out["dH"] * H.double().numpy()).sum())
    rhs = float((out["dW"] * W.double().numpy()).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), f"<dH,H>={lhs} != <dW,W>={rhs}"
    assert np.all(out["dH_abs"] >= np.abs(out["dH"])) and np.all(out["dW_abs"] >= np.abs(out["dW"]))


def pin_bwd_out_of_range_target(fwd, bwd):
    """A target outside [0, V) matches no vocabulary entry: that row's dH is
    g_i times the gradient of its lse (checked by finite differences of the
    forward's lse); other rows are unchanged."""
    rng = np.random.default_rng(44)
    N, D, V = 3, 4, 6
    Hn = (rng.standard_normal((N, D)) * 0.5).astype(np.float32)
    Wn = (rng.standard_normal((V, D)) * 0.5).astype(np.float32)
    g = np.array([0.75, 1.25, 0.5], np.float32)
    good = _y([1, 4, 2])
    bad = _y([-1, 4, 2])
    ob = bwd(_f32(Hn), _f32(Wn), bad, g)
    og = bwd(_f32(Hn), _f32(Wn), good, g)
    _close(ob["dH"][1:], og["dH"][1:], 0.0, "rows next to the bad target")

    def lse0(h):
        _, lse, _ = fwd(_f32(h), _f32(Wn), bad)
        return float(g[0]) * float(lse[0])

    fd = np.array([_richardson(lse0, Hn, (0, d), 2.0 ** -6) for d in range(D)])
    _close(ob["dH"][0], fd, 2e-6, "out-of-range row = g * d lse / d H")


def pin_bwd_rows_subset(fwd, bwd):
    """dH for a subset of rows, in any order, equals those rows of the full run."""
    rng = np.random.default_rng(45)
    N, D, V = 7, 8, 40
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)))
    y = _y(rng.integers(0, V, N))
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    full = bwd(H, W, y, g)
    sub = bwd(H, W, y, g, rows=[5, 0, 3], want_dW=False)
    _close(sub["dH"], full["dH"][[5, 0, 3]], 0.0, "row subset dH")


def pin_bwd_autograd(fwd, bwd):
    """Agreement with float64 reverse-mode differentiation of the definition in
    torch (an independent implementation of the same derivative)."""
    rng = np.random.default_rng(46)
    N, D, V = 6, 12, 37
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)))
    y = _y(rng.integers(0, V, N))
    g = rng.uniform(0.5, 1.5, N).astype(np.float32)
    out = bwd(H, W, y, g)
    Hd = H.double().clone().requires_grad_()
    Wd = W.double().clone().requires_grad_()
    Z = Hd @ Wd.T
    loss = torch.logsumexp(Z, dim=1) - Z.gather(1, y.long()[:, None])[:, 0]
    (loss * torch.as_tensor(g, dtype=torch.float64)).sum().backward()
    _close(out["dH"], Hd.grad.numpy(), 1e-13, "dH vs autograd")
    _close(out["dW"], Wd.grad.numpy(), 1e-13, "dW vs autograd")


# ------------------------------------------------------- sums of |terms| (two-sided)
# The backward's GPU tolerance is proportional to these sums, so they are
# pinned from both sides by closed forms: a sum that came out too large would
# loosen every backward check, one too small would fail correct results.
def pin_bwd_term_sums_single_word(fwd, bwd):
    """V = 1: the softmax is 1 and the one-hot is 1, so both terms of dZ_i0
    have size |g_i|: dH_abs_id = 2 |g_i| |W_0d| and dW_abs_0d = sum_i 2 |g_i| |H_id|
    (with g, H and W of both signs)."""
    rng = np.random.default_rng(47)
    N, D = 5, 9
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((1, D)))
    g = np.array([1.25, -0.5, 0.75, -2.0, 0.375], np.float32)
    out = bwd(H, W, _y([0] * N), g)
    Hd, Wd, gd = H.double().numpy(), W.double().numpy(), g.astype(np.float64)
    _close(out["dH_abs"], 2.0 * np.abs(gd)[:, None] * np.abs(Wd[0])[None, :], 1e-15, "V=1 dH_abs")
    _close(out["dW_abs"], (2.0 * np.abs(gd)[:, None] * np.abs(Hd)).sum(axis=0)[None, :], 1e-14, "V=1 dW_abs")


def pin_bwd_term_sums_signed_rows(fwd, bwd):
    """Vocabulary rows that differ only in the signs of their entries
    (|W_vd| = |w_d| for every v) give a non-uniform softmax, yet
    dH_abs_id = |g_i| |w_d| sum_v (p_iv + [v == y_i]) = 2 |g_i| |w_d| for a target
    in [0, V) (the softmax sums to 1, the one-hot to 1), and |g_i| |w_d| for a
    target outside [0, V) (an empty one-hot)."""
    rng = np.random.default_rng(48)
    N, D, V = 6, 10, 23
    w = rng.standard_normal(D)
    W = _bf16(rng.choice([-1.0, 1.0], size=(V, D)) * w[None, :])
    H = _bf16(rng.standard_normal((N, D)))
    yn = rng.integers(0, V, N)
    yn[2] = -1
    yn[4] = V
    g = rng.uniform(-1.5, 1.5, N).astype(np.float32)
    out = bwd(H, W, _y(yn), g)
    Wd = W.double().numpy()
    assert np.all(np.abs(Wd) == np.abs(Wd[0])[None, :]), "the rows must share their magnitudes"
    _, lse, _ = fwd(H, W, _y(yn))
    z = H.double().numpy() @ Wd.T
    assert np.ptp(z, axis=1).min() > 1.0, "the softmax must not be uniform"
    hits = np.where((yn >= 0) & (yn < V), 2.0, 1.0)
    want = hits[:, None] * np.abs(g.astype(np.float64))[:, None] * np.abs(Wd[0])[None, :]
    _close(out["dH_abs"], want, 1e-13, "signed rows dH_abs")


def pin_bwd_term_sums_columns(fwd, bwd):
    """For targets in [0, V), sum_v (p_iv + [v == y_i]) = 2 for every row, so each
    column of dW_abs sums over the vocabulary to 2 sum_i |g_i| |H_id|, whatever
    the inputs."""
    rng = np.random.default_rng(49)
    N, D, V = 7, 12, 40
    H = _bf16(rng.standard_normal((N, D)))
    W = _bf16(rng.standard_normal((V, D)) * 0.7)
    y = _y(rng.integers(0, V, N))
    g = rng.uniform(-1.0, 2.0, N).astype(np.float32)
    out = bwd(H, W, y, g)
    want = 2.0 * (np.abs(g.astype(np.float64))[:, None] * np.abs(H.double().numpy())).sum(axis=0)
    _close(out["dW_abs"].sum(axis=0), want, 1e-13, "column sums of dW_abs")


def pin_bwd_hand_examples(fwd, bwd):
    """Hand-worked gradients and term sizes stored in
    tests/golden/hand_examples_backward.json."""
    with open(os.path.join(GOLDEN, "hand_examples_backward.json")) as f:
        data = json.load(f)
    getcontext().prec = 50
    env = {"ln": lambda x: Decimal(x).ln(), "exp": lambda x: Decimal(x).exp(), "__builtins__": {}}

    def ev(expr):
        import re
        return float(eval(re.sub(r"(\d+(?:\.\d+)?)", r"Decimal('\1')", expr), {**env, "Decimal": Decimal}))

    for ex in data["examples"]:
        for mk in (_bf16, _f32):
            out = bwd(mk(ex["H"]), mk(ex["W"]), _y(ex["y"]), np.asarray(ex["g"], np.float32))
            for key in ("dH", "dW", "dH_abs", "dW_abs"):
                want = [[ev(e) for e in row] for row in ex[key]]
                _close(out[key], want, 1e-15, f"{ex['name']} {key}")


BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_zero_weights,
    pin_bwd_single_word,
    pin_bwd_identities,
    pin_bwd_out_of_range_target,
    pin_bwd_rows_subset,
    pin_bwd_autograd,
    pin_bwd_term_sums_single_word,
    pin_bwd_term_sums_signed_rows,
    pin_bwd_term_sums_columns,
    pin_bwd_hand_examples,
]
