"""HIP graph capture: flce_forward_ws, flce_backward, flce_forward_noalloc and
the quantised head's forward and backward enqueue kernel launches only (no
allocation, no memset), so a caller can capture them into a graph and replay
it. Each graph is replayed several times, with new inputs copied into its
static buffers by ordinary eager work between replays, and every replay must
equal the eager calls on the same inputs bit for bit.
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


def _replay_and_compare(step, load_inputs, outputs, want, what):
    """Warm up step() on a side stream, capture it, then replay it twice over
    every input set (copied in by eager work between replays), comparing every
    output with the eager result bit for bit."""
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
        for k in range(len(want)):
            load_inputs(k)
            for t in outputs:
                t.fill_(float("nan"))             # the replay must overwrite every output
            graph.replay()
            torch.cuda.synchronize()
            for i, (got, ref) in enumerate(zip(outputs, want[k])):
                same = torch.equal(got.view(torch.int32), ref.view(torch.int32))  # bit patterns (NaN rows too)
                assert same, f"{what}: replay {rep}, inputs {k}: output {i} differs from the eager call"


def test_noalloc_forward_replayed_from_a_graph():
    """flce_forward_noalloc is meant for callers under graph capture: captured
    and replayed, it equals flce_forward_ws on every input set."""
    import linear_cross_entropy_amd as flce
    N, D, V = 777, 256, 30001
    print(f"[graph noalloc] N={N} D={D} V={V} bf16", flush=True)
    inputs = [workloads.make_custom(N, D, V, "bf16", seed=71 + k, device=DEV) for k in range(3)]
    want = []
    for H, W, y in inputs:
        ws = flce.workspace(N, D, V, "bf16", DEV)
        loss = torch.empty(N, dtype=torch.float32, device=DEV)
        lse = torch.empty(N, dtype=torch.float32, device=DEV)
        flce.flce_forward_ws(H, W, y, ws, loss=loss, lse=lse)
        want.append((loss, lse))
    torch.cuda.synchronize()
    H_s, W_s, y_s = (t.clone() for t in inputs[0])
    loss = torch.empty(N, dtype=torch.float32, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)

    def load(k):
        for s, t in zip((H_s, W_s, y_s), inputs[k]):
            s.copy_(t)

    _replay_and_compare(lambda: flce.flce_forward_noalloc(H_s, W_s, y_s, loss=loss, lse=lse),
                        load, (loss, lse), want, "noalloc")


def test_quant_forward_and_backward_replayed_from_a_graph():
    """The quantised head's forward and frozen-head backward enqueue kernels
    only: three vocabulary slices (D = 16384, V = 13000), captured together
    and replayed over two heads."""
    import linear_cross_entropy_amd as flce
    N, D, V, bits, group = 64, 16384, 13000, 4, 64
    print(f"[graph quant] N={N} D={D} V={V} bits={bits} group={group}", flush=True)
    inputs = []
    for k in range(2):
        H, codes, scales, biases, y = workloads.make_quant(N, D, V, bits, group, seed=83 + k, device=DEV,
                                                           w_std=1.0 / D ** 0.5)
        y[0] = -1                                 # an ignored row: NaN loss, zero gradient
        g = torch.linspace(0.5, 1.5, N, dtype=torch.float32, device=DEV) * (k + 1)
        inputs.append((H, codes, scales, biases, y, g))
    ws_f = torch.empty(flce.flce_forward_quant_workspace_bytes(N, D, V, bits, group), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(flce.flce_backward_quant_workspace_bytes(N, D, V, bits, group), dtype=torch.uint8,
                       device=DEV)
    want = []
    for H, codes, scales, biases, y, g in inputs:
        loss, lse = flce.flce_forward_quant(H, codes, scales, biases, y, bits, group, workspace=ws_f)
        dH = flce.flce_backward_quant(H, codes, scales, biases, y, lse, g, bits, group, workspace=ws_b)
        want.append((loss, lse, dH))
    torch.cuda.synchronize()
    statics = [t.clone() for t in inputs[0]]
    loss = torch.empty(N, dtype=torch.float32, device=DEV)
    lse = torch.empty(N, dtype=torch.float32, device=DEV)
    dH = torch.empty(N, D, dtype=torch.float32, device=DEV)

    def step():
        H_s, c_s, s_s, b_s, y_s, g_s = statics
        flce.flce_forward_quant(H_s, c_s, s_s, b_s, y_s, bits, group, workspace=ws_f, loss=loss, lse=lse)
        flce.flce_backward_quant(H_s, c_s, s_s, b_s, y_s, lse, g_s, bits, group, workspace=ws_b, dH=dH)

    def load(k):
        for s, t in zip(statics, inputs[k]):
            s.copy_(t)

    _replay_and_compare(step, load, (loss, lse, dH), want, "quant")
