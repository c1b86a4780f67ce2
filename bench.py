#!/usr/bin/env python3
"""Benchmark of the fused linear cross-entropy forward on one MI355X.

One step = one full forward (the partials launch, then the merge launch) over
the workload's synthetic inputs, already resident in device memory. Prints one
JSON line:

  value        tokens/s over the K timed steps (N tokens per step)
  roofline     the partials kernel (the dominant launch) against the bf16
               dense matrix-core peak: achieved = 2*N*V*D FLOP / its average
               duration, measured with HIP events on the stream it runs on
  cpu_baseline the float64 CPU oracle on a bounded row sample of the same
               workload, on the host's cores (a reported baseline only)

After the W warm-up steps, untimed launches continue until the per-launch
time has settled (two consecutive 10-launch medians within 0.5%, at most
--settle-seconds), then exactly K steps are timed. The forward's line also
carries mfma_ceiling: the sustained rate of the same matrix-core instruction
with register operands, measured in the same run (libflce_ceiling.so), and,
for the production workload, also_measured: the backward, the 4-bit quantised
head's forward, the small and medium workloads, and cold-cache forwards
(--cold: a 512 MiB read before each timed launch), each timed the same way
with fewer steps (--no-extra leaves them out).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload prod_bf16]
       python bench.py --backward ...   (the backward instead: one step = one
       flce_backward, 3 x 2*N*V*D FLOP, timed over all of its launches)
       python bench.py --mfma-ceiling   (only the matrix-core ceiling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X dense peaks (TFLOP/s): bf16 matrix 2516.6 (256 CU x 2.4 GHz x
# 4096 FLOP/clk/CU), fp32 matrix 157.3.
PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0
COLD_SCRUB_BYTES = 512 << 20  # twice the 256 MB Infinity Cache
METRIC = "tokens/s + % bf16 MFMA peak, fused LCE fwd N=8192 D=4096 V=151936"
# The page's own number for this workload ("Een gefuseerde forward-kernel voor
# lineaire cross-entropy op Apple-GPU's", abstract and section 3): its fused
# MLX/Metal forward took 2.105 s for the 8192 tokens on one Apple M1 Max. It is
# another machine's figure, reported as context for vs_baseline, not a target.
PAGE_TOKENS_PER_S = 8192 / 2.105
PAGE_REF = ("the page's fused MLX/Metal forward on one Apple M1 Max: 8192 tokens in 2.105 s "
            "(3892 tokens/s); another machine, context only")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_flce_partials_prod_bf16.json")
# the kernels and the planners that choose their tiles and grids
KERNEL_SRC = (os.path.join(ROOT, "linear_cross_entropy_amd", "csrc", "flce.hip"),
              os.path.join(ROOT, "linear_cross_entropy_amd", "csrc", "flce_plan.h"))


def kernel_source_sha(paths=KERNEL_SRC) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that
    counters stay attached to the code they were taken on across comment edits."""
    import re
    if isinstance(paths, str):
        paths = (paths,)
    texts = []
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        texts.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(texts).encode()).hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per partials launch from the committed rocprofv3 counter runs,
    or None when they were taken on a different kernel source or workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha() or t.get("workload") != workload:
        return None
    return {"fetch_bytes": t["fetch_bytes_per_launch"], "write_bytes": t["write_bytes_per_launch"],
            "total_bytes": t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"],
            "copy_scale": t.get("copy_scale"), "source": os.path.relpath(TRAFFIC_FILE, ROOT),
            "what": "L2 fetches from and writes to the memory fabric per launch: an upper bound on HBM bytes "
                    "(Infinity Cache hits are not separable on this part); the algorithmic bytes are the lower bound"}


def cpu_baseline(H, W, y, w, target_seconds: float, max_rows: int):
    """Time the oracle on a row sample sized for about target_seconds of wall time."""
    import oracle
    import workloads
    Hc, Wc, yc = H.cpu(), W.cpu(), y.cpu()
    threads = oracle.num_threads()
    # calibrate on one row per thread, then size the sample
    probe = workloads.subset_rows(w.N, max(1, threads), seed=777).numpy()[:threads]
    t0 = time.perf_counter()
    oracle.forward(Hc, Wc, yc, rows=probe)
    t_probe = time.perf_counter() - t0
    per_row_wall = t_probe / len(probe)
    rows_n = int(max(len(probe), min(max_rows, target_seconds / max(per_row_wall, 1e-9))))
    rows_n = max(threads, (rows_n // threads) * threads)
    rows = workloads.subset_rows(w.N, rows_n, seed=778).numpy()
    t0 = time.perf_counter()
    oracle.forward(Hc, Wc, yc, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {w.N} rows (first/last {max(1, len(rows) // 8)} plus seeded "
                      f"random), each a full float64 row of {w.V} logits over D={w.D}; "
                      f"{dt:.2f} s wall",
            "seconds": dt, "rows": len(rows)}


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline_backward(H, W, y, g, w, target_seconds: float, max_rows: int):
    """The oracle's backward for a row sample (dH rows only: dW needs every row)."""
    import oracle
    import workloads
    Hc, Wc, yc, gc = H.cpu(), W.cpu(), y.cpu(), g.cpu()
    threads = oracle.num_threads()
    probe = workloads.subset_rows(w.N, max(1, threads), seed=777).numpy()[:threads]
    t0 = time.perf_counter()
    oracle.backward(Hc, Wc, yc, gc, rows=probe, want_dW=False)
    per_row = (time.perf_counter() - t0) / len(probe)
    rows_n = int(max(len(probe), min(max_rows, target_seconds / max(per_row, 1e-9))))
    rows_n = max(threads, (rows_n // threads) * threads)
    rows = workloads.subset_rows(w.N, rows_n, seed=778).numpy()
    t0 = time.perf_counter()
    oracle.backward(Hc, Wc, yc, gc, rows=rows, want_dW=False)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"dH for {len(rows)} of {w.N} rows (seeded), each recomputing a full float64 row "
                      f"of {w.V} logits over D={w.D} and summing V*D products; dW not included; "
                      f"{dt:.2f} s wall"}


def bench_backward(args, w):
    """One step = flce_backward over the workload (Z recomputed, dZ, dH, dW),
    with the forward's lse and a mean-over-tokens upstream gradient resident."""
    import torch
    import linear_cross_entropy_amd as flce
    import workloads
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.describe()}", file=sys.stderr, flush=True)
    H, W, y = workloads.make(w, dev)
    _, lse = flce.flce_forward(H, W, y)
    g = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=dev)
    dH = torch.empty(w.N, w.D, dtype=torch.float32, device=dev)
    dW = torch.empty(w.V, w.D, dtype=torch.float32, device=dev)
    ws = torch.empty(flce.flce_backward_workspace_bytes(w.N, w.D, w.V, w.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        flce.flce_backward(H, W, y, lse, g, workspace=ws, dH=dH, dW=dW, stream=stream)
    torch.cuda.synchronize()
    settled = settle(lambda: flce.flce_backward(H, W, y, lse, g, workspace=ws, dH=dH, dW=dW, stream=stream),
                     stream, args.settle_seconds, block=4)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} backward steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        flce.flce_backward(H, W, y, lse, g, workspace=ws, dH=dH, dW=dW, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    each = [a.elapsed_time(b) for a, b in ev]
    ms = sorted(each)
    avg = sum(ms) / len(ms)
    flops = 3 * w.flops
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / (avg * 1e-3) / 1e12
    result = {
        "metric": f"tokens/s + % {w.dtype} MFMA peak, fused LCE backward N={w.N} D={w.D} V={w.V}",
        "value": w.N * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, as the forward); upstream gradient 1/N per token",
        "config": {"workload": w.name, "N": w.N, "D": w.D, "V": w.V, "input_dtype": w.dtype,
                   "workspace_bytes": ws.numel()},
        "roofline": {
            "bound": "mfma",
            "kernel": "flce_backward (all launches: transposes, dZ pass, dH and dW products)",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": None,
            "algorithmic_flop_per_launch": flops,
            "algorithmic_bytes_per_launch": w.N * w.D * 2 + w.V * w.D * 2 + 12 * w.N + 4 * (w.N + w.V) * w.D,
            "kernel_ms_avg": avg,
            "kernel_ms_median": ms[len(ms) // 2],
            "kernel_ms_min": ms[0],
            "kernel_ms_each": [round(t, 4) for t in each],
        },
        "outputs_finite": bool(torch.isfinite(dH).all().item() and torch.isfinite(dW).all().item()),
        "settle": settled,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's backward on a row sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_backward(H, W, y, g, w, args.cpu_seconds, args.cpu_max_rows)
    else:
        result["cpu_baseline"] = None
    result["env"] = device_env()
    return result


def device_env():
    """What the line was measured on: ROCm (HIP) version, GPU architecture and
    compute-unit count as the runtime reports them, and the host threads the
    CPU oracle may use."""
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"hip": torch.version.hip, "torch": torch.__version__, "device": props.name,
            "arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "hbm_bytes": props.total_memory, "host_threads": os.cpu_count()}


def settle(launch, stream, seconds: float, block: int = 10, tol: float = 0.005):
    """Untimed launches after the warm-up steps until the part's clock has
    settled: blocks of `block` launches, each timed with HIP events on the
    launch stream, until two consecutive block medians agree within `tol`, or
    `seconds` have passed. (On a freshly leased part the first seconds of
    launches can run a few percent slow and speed up as the power manager
    settles.) Returns what was done, for the JSON line."""
    import torch
    t0 = time.perf_counter()
    medians = []
    n = 0
    while time.perf_counter() - t0 < seconds:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(block)]
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        n += block
        ms = sorted(a.elapsed_time(b) for a, b in ev)
        medians.append(ms[len(ms) // 2])
        if len(medians) >= 2 and abs(medians[-1] - medians[-2]) <= tol * medians[-2]:
            break
    return {"launches": n, "seconds": round(time.perf_counter() - t0, 3),
            "settled": len(medians) >= 2 and abs(medians[-1] - medians[-2]) <= tol * medians[-2],
            "block_medians_ms": [round(m, 4) for m in medians]}


def mfma_ceiling(seconds: float = 0.5, kind: str = "random", order: int = 0):
    """The sustained rate of v_mfma_f32_32x32x16_bf16 with operands in
    registers (libflce_ceiling.so), one workgroup of 8 waves per compute unit,
    and the shader clock it held (s_memtime against the 100 MHz s_memrealtime).
    Random operands toggle the datapath as real data does; constant ones show
    the clock the part reaches when they do not."""
    import torch
    from linear_cross_entropy_amd import ceiling
    dev = torch.device("cuda:0")
    grid, threads = torch.cuda.get_device_properties(0).multi_processor_count, 512
    n = grid * threads * 64
    gen = torch.Generator(device=dev).manual_seed(123)
    ops = (torch.randn(n, device=dev, generator=gen) if kind == "random"
           else torch.ones(n, device=dev)).to(torch.bfloat16)
    per_iter = grid * (threads // 64) * ceiling.MFMA_PER_ITER * ceiling.FLOP_PER_MFMA
    iters = 2000
    ceiling.flce_ceiling_mfma(ops, order, iters, grid, threads)        # warm-up and rate probe
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    ceiling.flce_ceiling_mfma(ops, order, iters, grid, threads)
    b.record()
    torch.cuda.synchronize()
    iters = max(iters, int(iters * seconds * 1e3 / max(a.elapsed_time(b), 1e-3)))
    a.record()
    _, clk = ceiling.flce_ceiling_mfma(ops, order, iters, grid, threads)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    c = clk.view(grid, 4).cpu().double()
    ghz = float(((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * 0.1).median())
    tflops = per_iter * iters / (ms * 1e-3) / 1e12
    return {"operands": kind, "instruction": CEILING_INSTRUCTION[order], "tflops": tflops,
            "frac_of_peak": tflops / PEAK_TFLOPS["bf16"], "shader_clock_ghz": ghz, "ms": ms,
            "kernel": f"flce_ceiling_kernel<{order}> (libflce_ceiling.so)"}


CEILING_INSTRUCTION = {0: "v_mfma_f32_32x32x16_bf16", 4: "v_mfma_f32_16x16x32_bf16"}


def bench_ceiling(args):
    """--mfma-ceiling: the matrix-core ceiling of both bf16 instruction forms
    with random operands (alternated twice), and of the 32x32x16 form with
    constant ones, one JSON line."""
    runs = {0: [], 4: []}
    for _ in range(2):
        for order in (0, 4):
            runs[order].append(mfma_ceiling(args.ceiling_seconds, "random", order))
    const = mfma_ceiling(args.ceiling_seconds, "const", 0)
    best = {o: max(r, key=lambda x: x["tflops"]) for o, r in runs.items()}
    print(json.dumps({
        "metric": "sustained bf16 MFMA rate, register operands",
        "value": best[4]["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic (random N(0,1) bf16 operand fragments; and all-ones)",
        "peak": PEAK_TFLOPS["bf16"],
        "random_32x32x16": runs[0], "random_16x16x32": runs[4], "constant_32x32x16": const,
        "env": device_env()}), flush=True)


def bench_quant(args, w):
    """The forward with a quantised head of the workload's shape: each step is
    one flce_forward_quant (dequantisation slice by slice, the partials kernel
    per slice, one merge), timed whole with HIP events on the launch stream.
    With --backward, each step is one flce_backward_quant (dH of the mean
    loss for the frozen head, given the forward's lse): 2 x 2 N V D FLOP."""
    import torch
    import linear_cross_entropy_amd as flce
    import workloads
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.describe()} with a {args.quant}-bit head, group {args.group}",
          file=sys.stderr, flush=True)
    H, codes, scales, biases, y = workloads.make_quant(w.N, w.D, w.V, args.quant, args.group, seed=w.index,
                                                       device=dev)
    ws = torch.empty(flce.flce_forward_quant_workspace_bytes(w.N, w.D, w.V, args.quant, args.group),
                     dtype=torch.uint8, device=dev)
    loss = torch.empty(w.N, device=dev)
    lse = torch.empty(w.N, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        flce.flce_forward_quant(H, codes, scales, biases, y, args.quant, args.group, workspace=ws,
                                loss=loss, lse=lse, stream=stream)

    flops = w.flops
    what = "fwd"
    kernel = "flce_forward_quant (all launches: dequantisation per slice, partials per slice, merge)"
    if args.backward:
        step()
        g = torch.full((w.N,), 1.0 / w.N, dtype=torch.float32, device=dev)
        dH = torch.empty(w.N, w.D, dtype=torch.float32, device=dev)
        ws = torch.empty(flce.flce_backward_quant_workspace_bytes(w.N, w.D, w.V, args.quant, args.group),
                         dtype=torch.uint8, device=dev)

        def step():
            flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, args.quant, args.group, workspace=ws,
                                     dH=dH, stream=stream)
        flops = 2 * w.flops
        what = "backward (dH, frozen head)"
        kernel = ("flce_backward_quant (all launches: per slice dequantisation, transpose, dZ pass, dH product; "
                  "partial-sum add)")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settled = settle(step, stream, args.settle_seconds, block=4)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    each = [a.elapsed_time(b) for a, b in ev]
    avg = sum(each) / len(each)
    achieved = flops / (avg * 1e-3) / 1e12
    head_bytes = codes.numel() + 2 * scales.numel() * 4
    result = {
        "metric": f"tokens/s + % bf16 MFMA peak, fused LCE {what} with a {args.quant}-bit head "
                  f"N={w.N} D={w.D} V={w.V}",
        "value": w.N * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded; H ~ N(0,1) bf16, uniform {args.quant}-bit codes, per-group scales and "
                f"biases for weights of spread ~0.02, uniform int32 targets)",
        "config": {"workload": w.name, "N": w.N, "D": w.D, "V": w.V, "bits": args.quant, "group": args.group,
                   "head_bytes": head_bytes, "workspace_bytes": ws.numel()},
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": achieved,
            "peak": PEAK_TFLOPS["bf16"],
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_TFLOPS["bf16"],
            "traffic": None,
            "algorithmic_flop_per_launch": flops,
            "kernel_ms_avg": avg,
            "kernel_ms_median": sorted(each)[len(each) // 2],
            "kernel_ms_min": min(each),
            "kernel_ms_each": [round(t, 4) for t in each],
        },
        "outputs_finite": bool(torch.isfinite(dH if args.backward else loss).all().item()),
        "cpu_baseline": None,
        "settle": settled,
    }
    result["env"] = device_env()
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prod_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle's row sample")
    ap.add_argument("--cpu-max-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter scaling), then exit")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (flce_backward, given the forward's lse) instead of the forward")
    ap.add_argument("--quant", type=int, default=0, choices=(0, 4, 8), metavar="BITS",
                    help="time flce_forward_quant (with --backward: flce_backward_quant) with a BITS-bit head "
                         "of the workload's shape instead")
    ap.add_argument("--group", type=int, default=64, help="weights per scale/bias group with --quant")
    ap.add_argument("--settle-seconds", type=float, default=4.0,
                    help="after the warm-up steps, untimed launches until consecutive 10-launch medians agree "
                         "within 0.5%% (at most this long)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="leave out the matrix-core ceiling measured beside the forward")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the matrix-core ceiling (random and constant operands)")
    ap.add_argument("--ceiling-seconds", type=float, default=1.0)
    ap.add_argument("--cold", action="store_true",
                    help="forward: scrub the caches (a 512 MiB read) before each timed launch")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the headline forward (no also_measured block)")
    ap.add_argument("--also-steps", type=int, default=10, help="timed steps of each also_measured configuration")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (the forward shards by rows with no "
              "communication, so N GPUs run N independent copies). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.mfma_ceiling:
        bench_ceiling(args)
        return

    import workloads

    w = workloads.WORKLOADS[args.workload]
    if args.quant:
        print(json.dumps(bench_quant(args, w)), flush=True)
        return
    if args.backward:
        print(json.dumps(bench_backward(args, w)), flush=True)
        return
    result = bench_forward(args, w)
    if not args.no_extra and w.name == "prod_bf16":
        result["also_measured"] = also_measured(args)
    print(json.dumps(result), flush=True)


# The other configurations timed in the default run, after the headline
# forward (each with its own warm-up and settle phase, fewer steps, no CPU
# baseline): (label, workload, backward?, quantised-head bits, cold caches?)
ALSO = (
    ("backward_prod_bf16", "prod_bf16", True, 0, False),
    ("forward_quant4_prod_bf16", "prod_bf16", False, 4, False),
    ("forward_small_bf16", "small_bf16", False, 0, False),
    ("forward_medium_bf16", "medium_bf16", False, 0, False),
    ("backward_small_bf16", "small_bf16", True, 0, False),
    ("backward_medium_bf16", "medium_bf16", True, 0, False),
    ("forward_prod_bf16_cold", "prod_bf16", False, 0, True),
    ("forward_small_bf16_cold", "small_bf16", False, 0, True),
)


def also_measured(args):
    """Compact lines for the configurations in ALSO: the same measurements as
    --backward, --quant 4 and --workload give, with the HIP-event kernel time
    and its fraction of the bf16 dense peak."""
    import workloads
    out = {}
    for label, wname, backward, bits, cold in ALSO:
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.settle_seconds = args.also_steps, 2, min(args.settle_seconds, 2.0)
        sub.no_cpu_baseline, sub.no_ceiling, sub.backward, sub.quant = True, True, backward, bits
        sub.cold = cold
        w = workloads.WORKLOADS[wname]
        print(f"[bench] also: {label}", file=sys.stderr, flush=True)
        if bits:
            r = bench_quant(sub, w)
        elif backward:
            r = bench_backward(sub, w)
        else:
            r = bench_forward(sub, w)
        rl = r["roofline"]
        out[label] = {"metric": r["metric"], "kernel": rl["kernel"], "steps": sub.steps,
                      "kernel_ms_avg": rl["kernel_ms_avg"], "kernel_ms_median": rl["kernel_ms_median"],
                      "achieved_tflops": rl["achieved"], "frac": rl["frac"], "tokens_per_s": r["value"],
                      "settled": r["settle"]["settled"], "outputs_finite": r["outputs_finite"]}
        if "tile_vocab" in r["config"]:
            out[label]["tile"] = f'{r["config"]["tile_vocab"]}x{r["config"]["tile_tokens"]}'
            out[label]["chunks"] = r["config"]["chunks"]
        if cold:
            out[label]["cold_caches"] = True
            del out[label]["tokens_per_s"]  # the wall clock includes the cache scrubs
    return out


def bench_forward(args, w):
    """One step = flce_partials + flce_merge over the workload; the partials
    launch is the timed kernel."""
    import torch
    import linear_cross_entropy_amd as flce
    import workloads
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.describe()}", file=sys.stderr, flush=True)
    H, W, y = workloads.make(w, dev)
    loss = torch.empty(w.N, device=dev)
    lse = torch.empty(w.N, device=dev)
    ws = flce.workspace(w.N, w.D, w.V, w.dtype, dev)
    plan = flce.flce_get_plan(w.N, w.D, w.V, w.dtype)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step():
        flce.flce_partials(H, W, y, ws, stream=stream)
        flce.flce_merge(y, w.D, w.V, w.dtype, ws, loss=loss, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settled = settle(step, stream, args.settle_seconds)
    print(f"[bench] settled after {settled['launches']} more launches ({settled['seconds']} s)",
          file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    # --cold: before each timed launch, read a 512 MiB buffer on the same
    # stream (a reduction over it), which evicts H and W from the L2s and the
    # 256 MB Infinity Cache without leaving dirty lines behind, so the launch
    # reads its inputs from HBM (the events time the launch only; the
    # wall-clock rate then includes the scrubs)
    cold = getattr(args, "cold", False)
    scrub = torch.ones(COLD_SCRUB_BYTES // 4, dtype=torch.float32, device=dev) if cold else None
    scrub_sink = []
    print(f"[bench] timing {args.steps} steps{' (cold caches)' if cold else ''}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        if cold:
            scrub_sink.append(scrub.sum())
        a.record(stream)
        flce.flce_partials(H, W, y, ws, stream=stream)
        b.record(stream)
        flce.flce_merge(y, w.D, w.V, w.dtype, ws, loss=loss, lse=lse, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    kernel_ms_sorted = sorted(kernel_ms)
    avg_ms = sum(kernel_ms) / len(kernel_ms)
    ms_per_step = wall * 1e3 / args.steps

    flops = w.flops
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = traffic_from_profile(w.name)
    sanity = bool(torch.isfinite(loss).all().item() and torch.isfinite(lse).all().item())

    result = {
        "metric": METRIC if w.name == "prod_bf16" else
        f"tokens/s + % {w.dtype} MFMA peak, fused LCE fwd N={w.N} D={w.D} V={w.V}",
        "value": w.N * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (w.N * args.steps / wall) / PAGE_TOKENS_PER_S if w.name == "prod_bf16" else None,
        "vs_baseline_ref": PAGE_REF if w.name == "prod_bf16" else None,
        "dtype": w.dtype,
        "data": w.recipe(),
        "config": {"workload": w.name, "N": w.N, "D": w.D, "V": w.V, "input_dtype": w.dtype,
                   "tile_vocab": plan["tile_vocab"], "tile_tokens": plan["tile_tokens"],
                   "chunks": plan["chunks"], "grid": plan["grid"],
                   "workspace_bytes": plan["workspace_bytes"], "cold_caches": cold},
        "mfma_fraction_of_step": flops / (ms_per_step * 1e-3) / 1e12 / peak,
        "roofline": {
            "bound": "mfma",
            "kernel": "flce_partials_kernel",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic["total_bytes"] if traffic else None,
            "traffic_detail": traffic,
            "algorithmic_bytes_per_launch": w.N * w.D * 2 + w.V * w.D * 2 + 4 * w.N,
            "algorithmic_flop_per_launch": flops,
            "kernel_ms_avg": avg_ms,
            "kernel_ms_median": kernel_ms_sorted[len(kernel_ms) // 2],
            "kernel_ms_min": kernel_ms_sorted[0],
            "kernel_ms_each": [round(t, 4) for t in kernel_ms],
        },
        "outputs_finite": sanity,
        "kernel_source_sha": kernel_source_sha(),
        "settle": settled,
    }
    if not args.no_ceiling:
        # the ceiling of the instruction the partials kernel runs: 16x16x32 on
        # the bf16 256- and 320-row tiles, 32x32x16 on the 384-row tile (and
        # the fp32 kernel's instruction is not measured here)
        order = 4 if (w.dtype == "bf16" and plan["tile_vocab"] in (256, 320)) else 0
        print("[bench] measuring the matrix-core ceiling", file=sys.stderr, flush=True)
        ceil = mfma_ceiling(0.4, "random", order)
        keys = ("instruction", "tflops", "frac_of_peak", "shader_clock_ghz", "kernel")
        result["mfma_ceiling"] = {k: ceil[k] for k in keys}
        result["mfma_ceiling"]["kernel_frac_of_ceiling"] = achieved / ceil["tflops"]
        other = mfma_ceiling(0.4, "random", 4 - order)
        result["mfma_ceiling"]["other_instruction"] = {k: other[k] for k in keys}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(H, W, y, w, args.cpu_seconds, args.cpu_max_rows)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    else:
        result["cpu_baseline"] = None
    result["env"] = device_env()
    return result


if __name__ == "__main__":
    main()
