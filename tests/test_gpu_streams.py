"""Stream semantics of the C ABI: every entry point enqueues its work on the
stream it is given (NULL: the default stream), and calls on different streams
may run at the same time as long as they share only H and W. The kernels are
deterministic, so results on any stream must equal, bit for bit, those of the
same call on the current stream.

Streams are created at the default priority.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_amd  # noqa: F401  (fails loudly if the library is missing)


def _same(got, want, what):
    for i, (a, b) in enumerate(zip(got, want)):
        assert torch.equal(a, b), f"{what}: output {i} differs from the current-stream result"


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_side_streams_concurrent_calls(dt):
    """Forward (library-allocated and caller workspaces) and backward on two
    side streams at once, sharing H and W, against the current stream."""
    import linear_cross_entropy_amd as flce
    N, D, V = (1000, 512, 20000) if dt == "bf16" else (300, 128, 3000)
    print(f"[streams] N={N} D={D} V={V} {dt}", flush=True)
    H, W, y = workloads.make_custom(N, D, V, dt, seed=31, device=DEV)
    g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV)
    loss0, lse0 = flce.flce_forward(H, W, y)
    dH0, dW0 = flce.flce_backward(H, W, y, lse0, g)
    torch.cuda.synchronize()
    want = (loss0, lse0, dH0, dW0)

    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    with torch.cuda.stream(s1):                  # outputs allocated on s1; the binding uses s1
        l1, e1 = flce.flce_forward(H, W, y)
        h1, w1 = flce.flce_backward(H, W, y, e1, g)
    with torch.cuda.stream(s2):
        ws = flce.workspace(N, D, V, dt, DEV)
        l2, e2 = flce.flce_forward_ws(H, W, y, ws)
        h2, w2 = flce.flce_backward(H, W, y, e2, g)
    cur.wait_stream(s1)
    cur.wait_stream(s2)
    torch.cuda.synchronize()
    _same((l1, e1, h1, w1), want, f"{dt} stream 1")
    _same((l2, e2, h2, w2), want, f"{dt} stream 2")


def test_explicit_stream_argument():
    """Outputs allocated on the current stream, work passed an explicit other
    stream (the caller orders the two); the partials/merge pair likewise."""
    import linear_cross_entropy_amd as flce
    N, D, V = 700, 256, 9000
    H, W, y = workloads.make_custom(N, D, V, "bf16", seed=37, device=DEV)
    loss0, lse0 = flce.flce_forward(H, W, y)
    torch.cuda.synchronize()
    loss = torch.empty(N, dtype=torch.float32, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)
    loss2 = torch.empty_like(loss)
    lse2 = torch.empty_like(lse)
    ws = flce.workspace(N, D, V, "bf16", DEV)
    cur = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    flce.flce_forward(H, W, y, loss=loss, lse=lse, stream=s)
    flce.flce_partials(H, W, y, ws, stream=s)
    flce.flce_merge(y, D, V, "bf16", ws, loss=loss2, lse=lse2, stream=s)
    cur.wait_stream(s)
    torch.cuda.synchronize()
    _same((loss, lse, loss2, lse2), (loss0, lse0, loss0, lse0), "explicit stream")
