"""The C-ABI library loads and exports every declared symbol; host-side
argument checks and planning (no GPU, no compute)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def flce():
    import linear_cross_entropy_amd as m
    return m


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["flce_forward", "flce_forward_ws", "flce_partials", "flce_merge",
              "flce_workspace_bytes", "flce_get_plan", "flce_status_string", "flce_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(flce):
    lib = ctypes.CDLL(flce.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in flce.h but not exported"
    assert sorted(flce.EXPORTED) == declared_functions()


def test_status_strings(flce):
    assert flce.flce_status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert flce.flce_status_string(code) not in ("", "unknown status")
    assert flce.flce_status_string(12345) == "unknown status"
    assert flce.flce_version() >= 100


def test_workspace_bytes_is_linear_in_N_not_NxV(flce):
    N, D, V = 8192, 4096, 151936
    ws = flce.flce_workspace_bytes(N, D, V, "bf16")
    plan = flce.flce_get_plan(N, D, V, "bf16")
    C = plan["chunks"]
    assert ws >= (2 * C + 1) * N * 4
    assert ws < (2 * C + 1) * N * 4 + 3 * 256
    assert ws < 0.01 * N * V * 4          # far below one fp32 logits matrix
    assert flce.flce_workspace_bytes(0, D, V, "bf16") == 0


def test_plan_production_shape(flce):
    p = flce.flce_get_plan(8192, 4096, 151936, "bf16")
    assert p["row_blocks"] == math.ceil(8192 / p["tile_tokens"])
    assert p["vocab_tiles"] == math.ceil(151936 / p["tile_vocab"])
    assert p["grid"] == p["row_blocks"] * p["chunks"]
    assert p["grid"] <= 256 or p["grid"] % 256 == 0
    if p["xcd_rows"]:
        assert (p["row_blocks"] // p["xcd_rows"]) * (p["chunks"] // p["xcd_chunks"]) == 8
    assert p["lds_bytes"] <= 160 * 1024


@pytest.mark.parametrize("shape", [(1, 8, 1), (3, 72, 31), (2048, 1024, 32000), (4096, 2048, 50257),
                                   (8192, 8192, 262144), (128, 64, 1024), (1, 4104, 257)])
def test_plan_covers_every_tile_once(flce, shape):
    """Chunks partition the vocabulary tiles; every (row block, chunk) has a workgroup."""
    N, D, V = shape
    p = flce.flce_get_plan(N, D, V, "bf16")
    T, C = p["vocab_tiles"], p["chunks"]
    base, rem = divmod(T, C)
    starts = [c * base + min(c, rem) for c in range(C)]
    counts = [base + (c < rem) for c in range(C)]
    assert starts[0] == 0 and starts[-1] + counts[-1] == T and min(counts) >= 1
    # the workgroup -> (row block, chunk) map used by the kernel is a bijection
    seen = set()
    for b in range(p["grid"]):
        if p["xcd_rows"]:
            x, j = b & 7, b >> 3
            gc = C // p["xcd_chunks"]
            rb = (x // gc) * p["xcd_rows"] + j // p["xcd_chunks"]
            ch = (x % gc) * p["xcd_chunks"] + j % p["xcd_chunks"]
        else:
            rb, ch = divmod(b, C)
        assert 0 <= rb < p["row_blocks"] and 0 <= ch < C
        seen.add((rb, ch))
    assert len(seen) == p["grid"] == p["row_blocks"] * C


def test_gpu_parity_shapes_exercise_every_tile(flce):
    """The GPU parity grid reaches every bf16 tile configuration the planner
    can choose, with ragged vocabulary in each."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from parity import BOUNDARY_SHAPES, EDGE
    import workloads
    shapes = [(N, D, V) for N, D, V, dt in EDGE if dt == "bf16"] + list(BOUNDARY_SHAPES)
    shapes += [(w.N, w.D, w.V) for w in workloads.WORKLOADS.values() if w.dtype == "bf16"]
    ragged = {}
    for N, D, V in shapes:
        p = flce.flce_get_plan(N, D, V, "bf16")
        ragged.setdefault(p["tile_vocab"], False)
        ragged[p["tile_vocab"]] |= V % p["tile_vocab"] != 0
    assert set(ragged) == {256, 320, 384}
    assert all(ragged.values())


def test_invalid_arguments_rejected_before_any_launch(flce):
    lib = flce._lib
    buf = ctypes.c_void_p(4096)       # never dereferenced: every call below fails validation first
    # bad sizes / dtype
    assert lib.flce_forward(buf, buf, buf, 4, 0, 10, 0, buf, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(buf, buf, buf, 4, 8, 0, 0, buf, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(buf, buf, buf, -1, 8, 10, 0, buf, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(buf, buf, buf, 4, 8, 10, 7, buf, None, None) == flce.FLCE_ERR_UNSUPPORTED
    # D * sizeof(elem) must be a multiple of 16
    assert lib.flce_forward(buf, buf, buf, 4, 12, 10, 0, buf, None, None) == flce.FLCE_ERR_UNSUPPORTED
    assert lib.flce_forward(buf, buf, buf, 4, 6, 10, 1, buf, None, None) == flce.FLCE_ERR_UNSUPPORTED
    # null and misaligned pointers
    assert lib.flce_forward(None, buf, buf, 4, 8, 10, 0, buf, None, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward(buf, buf, buf, 4, 8, 10, 0, None, None, None) == flce.FLCE_ERR_INVALID_ARG
    odd = ctypes.c_void_p(4096 + 8)
    assert lib.flce_forward(odd, buf, buf, 4, 8, 10, 0, buf, None, None) == flce.FLCE_ERR_INVALID_ARG
    # caller workspace too small or misaligned
    need = flce.flce_workspace_bytes(4, 8, 10, 0)
    assert lib.flce_forward_ws(buf, buf, buf, 4, 8, 10, 0, buf, None, buf, need - 1, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward_ws(buf, buf, buf, 4, 8, 10, 0, buf, None, odd, need + 64, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_forward_ws(buf, buf, buf, 4, 8, 10, 0, buf, None, None, need, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_partials(buf, buf, buf, 4, 8, 10, 0, buf, need - 1, None) == flce.FLCE_ERR_INVALID_ARG
    assert lib.flce_merge(buf, 4, 8, 10, 0, None, None, buf, need, None) == flce.FLCE_ERR_INVALID_ARG
    # N == 0 is a no-op that touches nothing
    assert lib.flce_forward(None, None, None, 0, 8, 10, 0, None, None, None) == flce.FLCE_OK
    assert lib.flce_forward_ws(None, None, None, 0, 8, 10, 0, None, None, None, 0, None) == flce.FLCE_OK


def test_backward_arguments_rejected_before_any_launch(flce):
    lib = flce._lib
    buf = ctypes.c_void_p(4096)       # never dereferenced: every call below fails validation first
    odd = ctypes.c_void_p(4096 + 8)
    need = flce.flce_backward_workspace_bytes(4, 8, 10, 0)
    assert need > 0

    def bwd(H=buf, W=buf, y=buf, lse=buf, g=buf, N=4, D=8, V=10, dt=0, dH=buf, dW=buf, ws=buf, nb=need):
        return lib.flce_backward(H, W, y, lse, g, N, D, V, dt, dH, dW, ws, nb, None)

    assert bwd(D=0) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(V=0) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(N=-1) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(dt=7) == flce.FLCE_ERR_UNSUPPORTED
    assert bwd(D=12) == flce.FLCE_ERR_UNSUPPORTED          # 24 bytes per bf16 row
    for name in ("H", "W", "y", "lse", "g", "dH", "dW", "ws"):
        assert bwd(**{name: None}) == flce.FLCE_ERR_INVALID_ARG, name
    assert bwd(H=odd) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(ws=odd) == flce.FLCE_ERR_INVALID_ARG
    assert bwd(dH=odd) == flce.FLCE_ERR_INVALID_ARG        # dH takes 16-byte stores
    assert bwd(nb=need - 1) == flce.FLCE_ERR_INVALID_ARG


DZ_BUDGET = 2 ** 30   # bytes of dZ (one slice of the vocabulary) a backward call holds at once


def _up(x, m):
    return (x + m - 1) // m * m


def _slice_rows(N, V, es, copies):
    """Vocabulary rows per slice: the largest balanced size whose dZ buffers
    (copies x Vsp x Np elements) fit the budget, in multiples of 6144 rows (or
    64 when the budget holds fewer)."""
    Np = _up(N, 64)
    cap = DZ_BUDGET // (Np * es * copies)
    gran = 6144 if cap >= 6144 else 64
    maxv = max(cap // gran * gran, 64)
    if V <= maxv:
        return V
    n = -(-V // maxv)
    return min(maxv, _up(-(-V // n), gran))


def test_backward_workspace_layout(flce):
    """The workspace holds W_s^T for one vocabulary slice, H^T, and dZ^T of
    that slice (for fp32 also its row-major dZ), each rounded to 64 elements
    and 256-byte aligned; where the bf16 dH product is split over the
    vocabulary, S partial N x D float32 sums."""
    splits = {}
    for N, D, V, dt, es in [(4, 8, 10, 0, 2), (128, 64, 1024, 1, 4), (8192, 4096, 151936, 0, 2),
                            (2048, 1024, 32000, 0, 2), (4096, 2048, 50257, 0, 2),
                            (5000, 64, 262144, 0, 2), (0, 8, 10, 0, 2), (5000, 64, 262144, 1, 4),
                            (0, 8, 10, 1, 4), (8192, 8192, 262144, 0, 2), (8192, 4096, 151936, 1, 4)]:
        Np = _up(N, 64)
        Vs = _slice_rows(N, V, es, 2 if dt == 1 else 1) if N else 0
        Vsp = _up(Vs, 64)
        want = (_up(D * Vsp * es, 256) + _up(D * Np * es, 256) + _up(Vsp * Np * es, 256)
                + (_up(Np * Vsp * es, 256) if dt == 1 else 0))
        got = flce.flce_backward_workspace_bytes(N, D, V, dt)
        S = [s for s in range(1, 17) if got == want + (_up(s * N * D * 4, 256) if s > 1 else 0)]
        assert S, (N, D, V, dt, got, want)
        assert S[0] == 1 or (dt == 0 and N > 0), (N, D, V, dt)
        splits[(N, D, V, dt)] = S[0]
    assert splits[(8192, 4096, 151936, 0)] == 1       # enough dH tiles to fill the chip alone
    assert splits[(2048, 1024, 32000, 0)] > 1        # 32 dH tiles: split over the vocabulary
    assert splits[(4, 8, 10, 0)] == 1                # too little K to split
    assert flce.flce_backward_workspace_bytes(4, 12, 10, 0) == 0   # unsupported D
    # the slicing itself: the production shape takes three slices, the stress shape five;
    # the GPU test of ragged rows and slices relies on 92160 (bf16) and 24576 (fp32)
    assert _slice_rows(8192, 151936, 2, 1) == 55296
    assert -(-262144 // _slice_rows(8192, 262144, 2, 1)) == 5
    assert _slice_rows(5000, 262144, 2, 1) == 92160 and _slice_rows(5000, 262144, 4, 2) == 24576


@pytest.mark.parametrize("N,D,V", [(8192, 4096, 151936), (8192, 8192, 262144), (65536, 4096, 151936),
                                   (262144, 4096, 151936), (5000, 64, 262144)])
@pytest.mark.parametrize("dt", [0, 1])
def test_backward_memory_is_bounded(flce, N, D, V, dt):
    """No O(N V) memory: the dZ the backward holds at once stays within the
    1 GiB budget whatever N and V are, so the workspace is at most one slice of
    W^T, H^T and the budget (the N x V fp32 logits of the production shape
    alone would be 4.98 GB)."""
    es = 2 if dt == 0 else 4
    Np = _up(N, 64)
    Vs = _slice_rows(N, V, es, 2 if dt == 1 else 1)
    Vsp = _up(Vs, 64)
    dz_bytes = Vsp * Np * es * (2 if dt == 1 else 1)
    assert dz_bytes <= DZ_BUDGET
    got = flce.flce_backward_workspace_bytes(N, D, V, dt)
    assert 0 < got <= D * Vsp * es + D * Np * es + DZ_BUDGET + 4 * 256
    assert got < 0.4 * N * V * 4


def test_python_binding_validates_shapes(flce):
    import torch
    H = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(10, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        flce.flce_forward(H, W, y)            # CPU tensors are refused
    with pytest.raises(ValueError):
        flce._check_inputs(H.cuda() if torch.cuda.is_available() else H, W, y)


def test_quant_arguments_rejected_before_any_launch(flce):
    lib = flce._lib
    buf = ctypes.c_void_p(4096)       # never dereferenced: every call below fails validation first
    odd = ctypes.c_void_p(4096 + 4)
    need = flce.flce_forward_quant_workspace_bytes(4, 64, 100, 8, 32)
    assert need > 0

    def q(H=buf, c=buf, s=buf, b=buf, y=buf, N=4, D=64, V=100, bits=8, group=32, loss=buf, lse=None,
          ws=buf, nb=need):
        return lib.flce_forward_quant(H, c, s, b, y, N, D, V, bits, group, loss, lse, ws, nb, None)

    assert q(bits=3) == flce.FLCE_ERR_UNSUPPORTED
    assert q(bits=16) == flce.FLCE_ERR_UNSUPPORTED
    assert q(group=12) == flce.FLCE_ERR_UNSUPPORTED        # not a multiple of 8
    assert q(group=128) == flce.FLCE_ERR_UNSUPPORTED       # does not divide D
    assert q(D=0) == flce.FLCE_ERR_INVALID_ARG
    assert q(N=-1) == flce.FLCE_ERR_INVALID_ARG
    for name in ("H", "c", "s", "b", "y", "loss", "ws"):
        assert q(**{name: None}) == flce.FLCE_ERR_INVALID_ARG, name
    assert q(c=odd) == flce.FLCE_ERR_INVALID_ARG           # codes need 16-byte alignment
    assert q(H=odd) == flce.FLCE_ERR_INVALID_ARG
    assert q(nb=need - 1) == flce.FLCE_ERR_INVALID_ARG
    assert q(N=0) == flce.FLCE_OK                          # nothing to do, nothing read


def test_quant_workspace_layout(flce):
    """One bf16 slice of Vs rows (a multiple of 3072, near 256 MiB) plus the
    partial states of every slice's chunks and the target logits."""
    def up(x, m=256):
        return (x + m - 1) // m * m

    for N, D, V in [(8192, 4096, 151936), (64, 16384, 13000), (300, 256, 5003), (7, 65536, 7000)]:
        vs = max(3072, int(256 * 2 ** 20 / (D * 2)) // 3072 * 3072)
        vs = min(vs, V)
        slices = -(-V // vs)
        last = V - (slices - 1) * vs
        C = (slices - 1) * flce.flce_get_plan(N, D, vs, "bf16")["chunks"] + \
            flce.flce_get_plan(N, D, last, "bf16")["chunks"]
        want = up(vs * D * 2) + 2 * up(C * N * 4) + up(N * 4)
        for bits, group in ((8, 64), (4, 128)):
            assert flce.flce_forward_quant_workspace_bytes(N, D, V, bits, group) == want, (N, D, V, bits)
    assert flce.flce_forward_quant_workspace_bytes(0, 64, 100, 8, 32) == 0


def test_quant_backward_arguments_rejected_before_any_launch(flce):
    lib = flce._lib
    buf = ctypes.c_void_p(4096)       # never dereferenced: every call below fails validation first
    odd = ctypes.c_void_p(4096 + 8)
    need = flce.flce_backward_quant_workspace_bytes(4, 64, 100, 8, 32)
    assert need > 0

    def qb(H=buf, c=buf, s=buf, b=buf, y=buf, lse=buf, g=buf, N=4, D=64, V=100, bits=8, group=32, dH=buf,
           ws=buf, nb=need):
        return lib.flce_backward_quant(H, c, s, b, y, lse, g, N, D, V, bits, group, dH, ws, nb, None)

    assert qb(bits=5) == flce.FLCE_ERR_UNSUPPORTED
    assert qb(group=20) == flce.FLCE_ERR_UNSUPPORTED
    for name in ("H", "c", "s", "b", "y", "lse", "g", "dH", "ws"):
        assert qb(**{name: None}) == flce.FLCE_ERR_INVALID_ARG, name
    assert qb(dH=odd) == flce.FLCE_ERR_INVALID_ARG         # 16-byte dH stores
    assert qb(nb=need - 1) == flce.FLCE_ERR_INVALID_ARG
    assert qb(N=0) == flce.FLCE_OK
    assert flce.flce_backward_quant_workspace_bytes(0, 64, 100, 8, 32) == 0
    # one dequantised slice, its transpose and dZ^T of the slice; the slices add
    # their dH products into dH in place, so no per-slice partial sums
    up = lambda x, m=256: (x + m - 1) // m * m
    N, D, V = 8192, 4096, 151936
    vs, Np = 30720, 8192
    base = up(vs * D * 2) + up(D * vs * 2) + up(vs * Np * 2)
    got = flce.flce_backward_quant_workspace_bytes(N, D, V, 4, 64)
    assert got == base                                     # five slices, no split within a slice
    # with many rows the slice shrinks so that its dZ^T stays within the budget
    N = 65536
    vs = _slice_rows(N, V, 2, 1)
    assert vs < 30720 and vs * N * 2 <= DZ_BUDGET
    got = flce.flce_backward_quant_workspace_bytes(N, D, V, 4, 64)
    assert got == up(vs * D * 2) + up(D * vs * 2) + up(vs * N * 2)


def test_header_is_plain_c_and_links(flce, tmp_path):
    """include/flce.h compiles as strict C11 (the boundary is meant for C
    callers, not only C++), and a C program that takes the address of every
    declared entry point links against the built library and runs the host-side
    ones (no GPU needed: planning, sizes, status text, version)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    names = declared_functions()
    lib_dir = os.path.dirname(flce.LIB_PATH)
    src = tmp_path / "uses_flce.c"
    src.write_text(
        '#include "flce.h"\n#include <stdio.h>\n'
        "typedef void (*any_fn)(void);\n"
        "static const any_fn entry_points[] = {\n"
        + "".join(f"  (any_fn){n},\n" for n in names)
        + "};\n"
        "int main(void) {\n"
        "  flce_plan_t plan;\n"
        "  int rc = flce_get_plan(8192, 4096, 151936, FLCE_BF16, &plan);\n"
        '  printf("%d %d %d %d %zu %s %d\\n", (int)(sizeof entry_points / sizeof entry_points[0]), rc,\n'
        "         plan.tile_vocab, plan.chunks, flce_workspace_bytes(8192, 4096, 151936, FLCE_BF16),\n"
        "         flce_status_string(FLCE_ERR_UNSUPPORTED), flce_version());\n"
        "  return 0;\n}\n")
    exe = tmp_path / "uses_flce"
    include_dir = os.path.dirname(HEADER)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-Wno-cast-function-type",
           "-I", include_dir, str(src), "-L", lib_dir, "-lflce", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    count, rc, tile, chunks, ws, *rest = out.stdout.split()
    plan = flce.flce_get_plan(8192, 4096, 151936, "bf16")
    assert int(count) == len(names) and int(rc) == 0
    assert int(tile) == plan["tile_vocab"] and int(chunks) == plan["chunks"]
    assert int(ws) == flce.flce_workspace_bytes(8192, 4096, 151936, "bf16")
    assert int(rest[-1]) == flce.flce_version()
