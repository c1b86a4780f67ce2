"""HIP graph capture: flce_forward_ws and flce_backward enqueue kernel launches
only (no allocation, no memset), so a caller can capture them into a graph and
replay it. The graph is replayed several times, with new inputs copied into
its static buffers by ordinary eager work between replays, and every replay
must equal the eager calls on the same inputs bit for bit.
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


def test_forward_and_backward_replayed_from_a_graph():
    import linear_cross_entropy_amd as flce
    N, D, V = 1000, 512, 20000
    print(f"[graph] N={N} D={D} V={V} bf16", flush=True)
    inputs = []
    for k in range(3):
        H, W, y = workloads.make_custom(N, D, V, "bf16", seed=41 + k, device=DEV)
        g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV) * (k + 1)
        inputs.append((H, W, y, g))

    # eager results for each input set
    want = []
    for H, W, y, g in inputs:
        loss, lse = flce.flce_forward(H, W, y)
        dH, dW = flce.flce_backward(H, W, y, lse, g)
        want.append((loss, lse, dH, dW))
    torch.cuda.synchronize()

    # static buffers the graph reads and writes
    H_s, W_s, y_s, g_s = (t.clone() for t in inputs[0])
    ws_f = flce.workspace(N, D, V, "bf16", DEV)
    ws_b = torch.empty(flce.flce_backward_workspace_bytes(N, D, V, "bf16"), dtype=torch.uint8, device=DEV)
    loss = torch.empty(N, dtype=torch.float32, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)
    dH = torch.empty(N, D, dtype=torch.float32, device=DEV)
    dW = torch.empty(V, D, dtype=torch.float32, device=DEV)

    def step():
        flce.flce_forward_ws(H_s, W_s, y_s, ws_f, loss=loss, lse=lse)
        flce.flce_backward(H_s, W_s, y_s, lse, g_s, workspace=ws_b, dH=dH, dW=dW)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(2):
        for k, (H, W, y, g) in enumerate(inputs):
            H_s.copy_(H)
            W_s.copy_(W)
            y_s.copy_(y)
            g_s.copy_(g)
            loss.fill_(float("nan"))              # the replay must overwrite every output
            dH.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for name, got, ref in zip(("loss", "lse", "dH", "dW"), (loss, lse, dH, dW), want[k]):
                assert torch.equal(got, ref), f"replay {rep}, inputs {k}: {name} differs from the eager call"
