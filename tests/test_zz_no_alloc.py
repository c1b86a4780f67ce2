"""flce_forward_noalloc (the forward for callers that cannot allocate: its
workspace is the library's static per-GPU scratch) against the existing
flce_forward_ws on the same inputs, through the C ABI: two calls in a row,
the second on a smaller input (the scratch then holds the first call's
partials, which the second must not read), and a shape too large for the
scratch, which must be refused with nothing enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def flce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd as m
    return m


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _noalloc(flce, H, W, y, loss, lse, stream):
    N, D = H.shape
    V = W.shape[0]
    dt = flce.FLCE_BF16 if H.dtype == torch.bfloat16 else flce.FLCE_FP32
    return flce._lib.flce_forward_noalloc(_p(H), _p(W), _p(y), N, D, V, dt, _p(loss), _p(lse),
                                          ctypes.c_void_p(stream.cuda_stream))


def _ws(flce, H, W, y, loss, lse, stream):
    N, D = H.shape
    V = W.shape[0]
    dt = flce.FLCE_BF16 if H.dtype == torch.bfloat16 else flce.FLCE_FP32
    nb = flce.flce_workspace_bytes(N, D, V, dt)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    rc = flce._lib.flce_forward_ws(_p(H), _p(W), _p(y), N, D, V, dt, _p(loss), _p(lse), _p(ws), nb,
                                   ctypes.c_void_p(stream.cuda_stream))
    return rc, ws


@pytest.mark.parametrize("first,second", [((8192, 4096, 151936, "bf16"), (300, 256, 5003, "bf16")),
                                          ((2048, 1024, 32001, "bf16"), (128, 64, 1024, "fp32"))])
def test_noalloc_matches_forward_ws_twice(flce, first, second):
    stream = torch.cuda.current_stream(DEV)
    for k, (N, D, V, dt) in enumerate((first, second)):
        print(f"[noalloc] call {k}: N={N} D={D} V={V} {dt}", flush=True)
        H, W, y = workloads.make_custom(N, D, V, dt, seed=40 + k, device=DEV)
        y[0] = -1                                          # an ignored row: NaN loss, valid lse
        loss_a = torch.full((N,), 7.0, device=DEV)
        lse_a = torch.full((N,), 7.0, device=DEV)
        loss_b = torch.full((N,), -7.0, device=DEV)
        lse_b = torch.full((N,), -7.0, device=DEV)
        rc, ws = _ws(flce, H, W, y, loss_a, lse_a, stream)
        assert rc == flce.FLCE_OK
        assert _noalloc(flce, H, W, y, loss_b, lse_b, stream) == flce.FLCE_OK
        torch.cuda.synchronize()
        la, sa, lb, sb = (t.cpu().numpy() for t in (loss_a, lse_a, loss_b, lse_b))
        assert np.isnan(la[0]) and np.isnan(lb[0])
        assert np.array_equal(la, lb, equal_nan=True), f"loss differs from flce_forward_ws (call {k})"
        assert np.array_equal(sa, sb), f"lse differs from flce_forward_ws (call {k})"
        assert np.isfinite(sb).all()


def test_noalloc_refuses_shapes_beyond_the_scratch(flce):
    """N = 2^22 tokens at the production head needs ~50 MB of partials: refused
    before anything is launched (outputs untouched)."""
    N, D, V = 1 << 22, 4096, 151936
    assert flce.flce_workspace_bytes(N, D, V, flce.FLCE_BF16) > (16 << 20)
    H = torch.zeros(16, dtype=torch.bfloat16, device=DEV)   # never read: the call fails first
    y = torch.zeros(16, dtype=torch.int32, device=DEV)
    out = torch.full((16,), 3.0, device=DEV)
    rc = flce._lib.flce_forward_noalloc(_p(H), _p(H), _p(y), N, D, V, flce.FLCE_BF16, _p(out), _p(out),
                                        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert rc == flce.FLCE_ERR_SCRATCH
    assert "scratch" in flce.flce_status_string(rc)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
