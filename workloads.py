"""Seeded synthetic inputs for the fused linear cross-entropy forward.

This module only draws inputs: hidden states H (N x D), an output projection W
(V x D) and int32 targets y (N). It holds none of the method's arithmetic, so
the CPU oracle, the tests and the benchmark can all use it without sharing any
computation with the HIP path.

The five named workloads are the production case the page "Een gefuseerde
forward-kernel voor lineaire cross-entropy op Apple-GPU's" measures (abstract and section 3:
N=8192, V=151936, D=4096, bfloat16 inputs) and smaller, odd-V and
larger-vocabulary variants of it, with the value distributions stated below.
No public dataset is involved.

Recipe:
  * Values are drawn in fp32 from a torch.Generator on the device the tensors
    live on, seeded with 1000*config_index + stream (H=0, W=1, targets=2,
    outlier rows=3), then rounded once to the input dtype with
    round-to-nearest-even (torch's ``.to(torch.bfloat16)``). Both paths read
    the same rounded bits.
  * "N(0, s)" means standard deviation s.
  * Targets are drawn on the CPU (they are small) and moved to the device.
    "zipf" means a truncated Zipf law P(y=k) proportional to (k+1)^-1.1 over
    k in [0, V), sampled by inverse CDF.
  * The large-vocabulary stress workload multiplies 64 distinct seeded W rows
    by 50 before rounding.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    N: int
    D: int
    V: int
    dtype: str            # "bf16" or "fp32"
    h_std: float
    w_std: float
    targets: str          # "uniform" or "zipf"
    outlier_rows: int = 0
    outlier_scale: float = 1.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def flops(self) -> float:
        return 2.0 * self.N * self.V * self.D

    def describe(self) -> str:
        return f"{self.name}: N={self.N} D={self.D} V={self.V} {self.dtype}"

    def recipe(self) -> str:
        """How the inputs are drawn, in words."""
        cast = "rounded to bf16" if self.dtype == "bf16" else "kept fp32"
        w = f"W ~ N(0,{self.w_std:g})"
        if self.outlier_rows:
            w += f" with {self.outlier_rows} seeded rows x{self.outlier_scale:g}"
        y = "Zipf(1.1) int32 targets" if self.targets == "zipf" else "uniform int32 targets"
        return f"synthetic (seeded; H ~ N(0,{self.h_std:g}), {w}, {cast}, {y})"


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 0, 128, 64, 1024, "fp32", 1.0 / 8.0, 1.0 / 8.0, "uniform"),
        Workload("small_bf16", 1, 2048, 1024, 32000, "bf16", 1.0, 0.02, "uniform"),
        Workload("medium_bf16", 2, 4096, 2048, 50257, "bf16", 1.0, 0.02, "zipf"),
        Workload("prod_bf16", 3, 8192, 4096, 151936, "bf16", 1.0, 0.02, "uniform"),
        Workload("stress_bf16", 4, 8192, 8192, 262144, "bf16", 1.0, 0.02, "uniform",
                 outlier_rows=64, outlier_scale=50.0),
    ]
}

STREAM_H, STREAM_W, STREAM_Y, STREAM_OUTLIER = 0, 1, 2, 3


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_matrix(rows: int, cols: int, std: float, dtype: torch.dtype, device, seed: int,
                  scale_rows: torch.Tensor | None = None, scale: float = 1.0,
                  chunk_rows: int = 16384) -> torch.Tensor:
    """rows x cols matrix of N(0, std) fp32 draws, rounded once to ``dtype``.

    Drawn in row chunks so that the fp32 staging never exceeds
    chunk_rows*cols*4 bytes; rows listed in ``scale_rows`` are multiplied by
    ``scale`` before rounding.
    """
    out = torch.empty(rows, cols, dtype=dtype, device=device)
    g = _gen(device, seed)
    sel = None
    if scale_rows is not None and scale_rows.numel():
        sel = torch.zeros(rows, dtype=torch.bool)
        sel[scale_rows] = True
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn(r1 - r0, cols, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        if sel is not None:
            local = torch.nonzero(sel[r0:r1]).flatten()
            if local.numel():
                x[local.to(device)] *= scale
        out[r0:r1] = x.to(dtype)
    return out


def targets(N: int, V: int, kind: str, seed: int) -> torch.Tensor:
    """int32 targets in [0, V), drawn on the CPU."""
    g = _gen("cpu", seed)
    if kind == "uniform":
        return torch.randint(0, V, (N,), generator=g, dtype=torch.int64).to(torch.int32)
    if kind == "zipf":
        k = torch.arange(1, V + 1, dtype=torch.float64)
        p = k.pow(-1.1)
        cdf = torch.cumsum(p, 0)
        cdf /= cdf[-1].clone()
        u = torch.rand(N, generator=g, dtype=torch.float64)
        y = torch.searchsorted(cdf, u, right=False).clamp_(max=V - 1)
        return y.to(torch.int32)
    raise ValueError(f"unknown target law {kind!r}")


def outlier_rows(V: int, count: int, seed: int) -> torch.Tensor:
    g = _gen("cpu", seed)
    return torch.randperm(V, generator=g)[:count]


def make(w: Workload | str, device="cpu"):
    """Return (H, W, y) for a named workload on ``device``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    base = 1000 * w.index
    H = normal_matrix(w.N, w.D, w.h_std, w.torch_dtype, device, base + STREAM_H)
    orows = outlier_rows(w.V, w.outlier_rows, base + STREAM_OUTLIER) if w.outlier_rows else None
    W = normal_matrix(w.V, w.D, w.w_std, w.torch_dtype, device, base + STREAM_W,
                      scale_rows=orows, scale=w.outlier_scale)
    y = targets(w.N, w.V, w.targets, base + STREAM_Y).to(device)
    return H, W, y


def make_custom(N: int, D: int, V: int, dtype: str = "bf16", seed: int = 0, device="cpu",
                h_std: float = 1.0, w_std: float = 0.02, target_kind: str = "uniform"):
    """Seeded inputs of an arbitrary shape (edge cases, ragged tails)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    base = 7919 * (seed + 1)
    H = normal_matrix(N, D, h_std, tdt, device, base + STREAM_H)
    W = normal_matrix(V, D, w_std, tdt, device, base + STREAM_W)
    y = targets(N, V, target_kind, base + STREAM_Y).to(device) if V > 0 else \
        torch.zeros(N, dtype=torch.int32, device=device)
    return H, W, y


STREAM_CODES, STREAM_SCALES, STREAM_BIASES = 4, 5, 6


def make_quant(N: int, D: int, V: int, bits: int, group: int, seed: int = 0, device="cpu",
               w_std: float = 0.02, target_kind: str = "uniform"):
    """Seeded inputs for a quantised head: H (N x D, bf16, N(0,1)), codes
    uniform over [0, 2^bits) stored as uint8 (V x D at 8 bits, V x D/2 at 4
    bits: byte b holds code 2b in its low nibble and 2b+1 in its high one),
    float32 scales and biases per group of ``group`` weights (V x D/group),
    and int32 targets. Scales are w_std * sqrt(12) / 2^bits times U(0.5, 1.5)
    and biases minus scale * (2^bits - 1) / 2 times U(0.9, 1.1), so that the
    weights they describe are centred with a spread of about w_std."""
    base = 7919 * (seed + 1)
    H = normal_matrix(N, D, 1.0, torch.bfloat16, device, base + STREAM_H)
    levels = 1 << bits
    g = _gen(device, base + STREAM_CODES)
    q = torch.randint(0, levels, (V, D), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    codes = q if bits == 8 else (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()
    G = D // group
    gs = _gen(device, base + STREAM_SCALES)
    scale = (torch.rand(V, G, generator=gs, device=device) + 0.5) * (w_std * 12.0 ** 0.5 / levels)
    gb = _gen(device, base + STREAM_BIASES)
    bias = -scale * ((levels - 1) / 2.0) * (torch.rand(V, G, generator=gb, device=device) * 0.2 + 0.9)
    y = targets(N, V, target_kind, base + STREAM_Y).to(device)
    return H, codes, scale.contiguous(), bias.contiguous(), y


def subset_rows(N: int, count: int = 256, seed: int = 12345) -> torch.Tensor:
    """Row sample used where the oracle cannot take every row: the first and
    last count//8 rows plus seeded random rows in between (sorted, unique)."""
    if N <= count:
        return torch.arange(N, dtype=torch.int64)
    edge = max(1, count // 8)
    head = torch.arange(0, edge)
    tail = torch.arange(N - edge, N)
    g = _gen("cpu", seed)
    mid = torch.randperm(N - 2 * edge, generator=g)[: count - 2 * edge] + edge
    return torch.unique(torch.cat([head, tail, mid])).to(torch.int64)
