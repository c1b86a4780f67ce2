"""Python binding of libflce.so, the fused linear cross-entropy forward (and
its backward) for AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/flce.h``. PyTorch supplies the
device memory and the stream. The functions keep the C names:

    flce_forward(H, W, targets, loss=None, lse=None, stream=None) -> (loss, lse)
    flce_forward_ws(H, W, targets, workspace, loss=None, lse=None, stream=None)
    flce_forward_noalloc(H, W, targets, loss=None, lse=None, stream=None)
    flce_partials(H, W, targets, workspace, stream=None)
    flce_merge(targets, D, V, dtype, workspace, loss=None, lse=None, stream=None)
    flce_workspace_bytes(N, D, V, dtype) -> int
    flce_get_plan(N, D, V, dtype) -> dict
    flce_backward(H, W, targets, lse, grad_loss, workspace=None, dH=None, dW=None, stream=None)
    flce_backward_workspace_bytes(N, D, V, dtype) -> int
    flce_status_string(status) -> str
    flce_version() -> int
    linear_cross_entropy(H, W, targets) -> loss   (torch.autograd: gradients for H and W)
    flce_forward_quant(H, codes, scales, biases, targets, bits, group, workspace=None, loss=None, lse=None, stream=None)
    flce_forward_quant_workspace_bytes(N, D, V, bits, group) -> int
    flce_backward_quant(H, codes, scales, biases, targets, lse, grad_loss, bits, group, workspace=None, dH=None, stream=None)
    flce_backward_quant_workspace_bytes(N, D, V, bits, group) -> int
    linear_cross_entropy_quant(H, codes, scales, biases, targets, bits, group) -> loss   (gradient for H)

The operation (page "Een gefuseerde forward-kernel
voor lineaire cross-entropy op Apple-GPU's", section 1): with logits Z = H W^T, lse_i = logsumexp(Z_i) and
loss_i = lse_i - Z[i, y_i], both fp32 per token.

If the library has not been built, importing this package raises: there is
no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflce.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python linear_cross_entropy_amd/_build.py`")

_lib = ctypes.CDLL(LIB_PATH)

FLCE_BF16 = 0
FLCE_FP32 = 1
FLCE_OK = 0
FLCE_ERR_INVALID_ARG = -1
FLCE_ERR_UNSUPPORTED = -2
FLCE_ERR_HIP = -3
FLCE_ERR_OOM = -4
FLCE_ERR_SCRATCH = -5

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

_lib.flce_forward.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]
_lib.flce_forward.restype = _i32
_lib.flce_forward_ws.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.flce_forward_ws.restype = _i32
_lib.flce_forward_noalloc.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp]
_lib.flce_forward_noalloc.restype = _i32
_lib.flce_partials.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]
_lib.flce_partials.restype = _i32
_lib.flce_merge.argtypes = [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.flce_merge.restype = _i32
_lib.flce_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
_lib.flce_workspace_bytes.restype = _sz
_lib.flce_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.flce_backward.restype = _i32
_lib.flce_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
_lib.flce_backward_workspace_bytes.restype = _sz
_lib.flce_forward_quant.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.flce_forward_quant.restype = _i32
_lib.flce_forward_quant_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i32]
_lib.flce_forward_quant_workspace_bytes.restype = _sz
_lib.flce_backward_quant.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _sz,
                                     _vp]
_lib.flce_backward_quant.restype = _i32
_lib.flce_backward_quant_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i32]
_lib.flce_backward_quant_workspace_bytes.restype = _sz
_lib.flce_status_string.argtypes = [_i32]
_lib.flce_status_string.restype = ctypes.c_char_p
_lib.flce_version.argtypes = []
_lib.flce_version.restype = _i32


class FlcePlan(ctypes.Structure):
    _fields_ = [
        ("tile_vocab", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
        ("row_blocks", ctypes.c_int32), ("vocab_tiles", ctypes.c_int32),
        ("chunks", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("xcd_rows", ctypes.c_int32), ("xcd_chunks", ctypes.c_int32),
        ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib.flce_get_plan.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(FlcePlan)]
_lib.flce_get_plan.restype = _i32

EXPORTED = ["flce_forward", "flce_forward_ws", "flce_forward_noalloc", "flce_partials", "flce_merge",
            "flce_workspace_bytes", "flce_get_plan", "flce_status_string", "flce_version",
            "flce_backward", "flce_backward_workspace_bytes",
            "flce_forward_quant", "flce_forward_quant_workspace_bytes",
            "flce_backward_quant", "flce_backward_quant_workspace_bytes"]


class FlceError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {flce_status_string(status)} (status {status})")
        self.status = status


def flce_status_string(status: int) -> str:
    return _lib.flce_status_string(int(status)).decode()


def flce_version() -> int:
    return int(_lib.flce_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FLCE_BF16
    if t.dtype == torch.float32:
        return FLCE_FP32
    raise ValueError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dtype_arg(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if dtype in (torch.bfloat16, "bf16"):
        return FLCE_BF16
    if dtype in (torch.float32, "fp32"):
        return FLCE_FP32
    raise ValueError(f"unsupported dtype {dtype!r}")


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_inputs(H, W, targets):
    for name, t in (("H", H), ("W", W), ("targets", targets)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if H.dim() != 2 or W.dim() != 2 or targets.dim() != 1:
        raise ValueError("H must be (N, D), W (V, D), targets (N,)")
    if H.shape[1] != W.shape[1] or targets.shape[0] != H.shape[0]:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)}, W {tuple(W.shape)}, targets {tuple(targets.shape)}")
    if H.dtype != W.dtype:
        raise ValueError("H and W must share a dtype")
    if targets.dtype != torch.int32:
        raise ValueError("targets must be int32")
    if not (H.device == W.device == targets.device):
        raise ValueError("H, W and targets must be on the same device")
    return H.shape[0], H.shape[1], W.shape[0], _dtype_code(H)


def _out(t, N, device, name):
    if t is None:
        return torch.empty(N, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or t.shape != (N,) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 ({N},) tensor on {device}")
    return t


def _ptr(t):
    return t.data_ptr() if t is not None else None


def flce_workspace_bytes(N: int, D: int, V: int, dtype) -> int:
    return int(_lib.flce_workspace_bytes(N, D, V, _dtype_arg(dtype)))


def flce_get_plan(N: int, D: int, V: int, dtype) -> dict:
    p = FlcePlan()
    rc = _lib.flce_get_plan(N, D, V, _dtype_arg(dtype), ctypes.byref(p))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_get_plan")
    return {name: getattr(p, name) for name, _ in FlcePlan._fields_}


def flce_forward(H, W, targets, loss=None, lse=None, stream=None, want_lse=True):
    """loss (and lse) per token; the workspace is allocated stream-ordered by the library."""
    N, D, V, dt = _check_inputs(H, W, targets)
    loss = _out(loss, N, H.device, "loss")
    if want_lse:
        lse = _out(lse, N, H.device, "lse")
    rc = _lib.flce_forward(_ptr(H), _ptr(W), _ptr(targets), N, D, V, dt, _ptr(loss),
                           _ptr(lse) if want_lse else None, _stream_ptr(stream, H.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward")
    return loss, (lse if want_lse else None)


def workspace(N: int, D: int, V: int, dtype, device) -> torch.Tensor:
    """A device buffer of flce_workspace_bytes for the shape (256-byte aligned)."""
    nbytes = max(1, flce_workspace_bytes(N, D, V, dtype))
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def flce_forward_ws(H, W, targets, ws, loss=None, lse=None, stream=None, want_lse=True):
    N, D, V, dt = _check_inputs(H, W, targets)
    loss = _out(loss, N, H.device, "loss")
    if want_lse:
        lse = _out(lse, N, H.device, "lse")
    rc = _lib.flce_forward_ws(_ptr(H), _ptr(W), _ptr(targets), N, D, V, dt, _ptr(loss),
                              _ptr(lse) if want_lse else None, _ptr(ws), ws.numel() * ws.element_size(),
                              _stream_ptr(stream, H.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward_ws")
    return loss, (lse if want_lse else None)


def flce_forward_noalloc(H, W, targets, loss=None, lse=None, stream=None):
    """flce_forward with the library's static scratch as workspace: the C call
    allocates nothing (outputs not given are allocated here, by torch).
    Shapes needing more than 16 MiB of workspace raise FlceError
    (FLCE_ERR_SCRATCH); calls on one GPU must not overlap."""
    N, D, V, dt = _check_inputs(H, W, targets)
    loss = _out(loss, N, H.device, "loss")
    lse = _out(lse, N, H.device, "lse")
    rc = _lib.flce_forward_noalloc(_ptr(H), _ptr(W), _ptr(targets), N, D, V, dt, _ptr(loss), _ptr(lse),
                                   _stream_ptr(stream, H.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward_noalloc")
    return loss, lse


def flce_partials(H, W, targets, ws, stream=None):
    N, D, V, dt = _check_inputs(H, W, targets)
    rc = _lib.flce_partials(_ptr(H), _ptr(W), _ptr(targets), N, D, V, dt, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream_ptr(stream, H.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_partials")


def flce_merge(targets, D: int, V: int, dtype, ws, loss=None, lse=None, stream=None):
    N = targets.shape[0]
    loss = _out(loss, N, targets.device, "loss")
    lse = _out(lse, N, targets.device, "lse")
    rc = _lib.flce_merge(_ptr(targets), N, D, V, _dtype_arg(dtype), _ptr(loss), _ptr(lse), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream_ptr(stream, targets.device))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_merge")
    return loss, lse


def flce_backward_workspace_bytes(N: int, D: int, V: int, dtype) -> int:
    return int(_lib.flce_backward_workspace_bytes(N, D, V, _dtype_arg(dtype)))


def _vec(t, N, device, name):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.shape != (N,) \
            or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 ({N},) tensor on {device}")
    return t


def _mat(t, rows, cols, device, name):
    if t is None:
        return torch.empty(rows, cols, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or t.shape != (rows, cols) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 ({rows}, {cols}) tensor on {device}")
    return t


def flce_backward(H, W, targets, lse, grad_loss, workspace=None, dH=None, dW=None, stream=None):
    """(dH, dW) = gradients of sum_i grad_loss[i] * loss_i, float32; lse is the
    forward's lse for the same inputs. The workspace (flce_backward_workspace_bytes)
    is allocated here when not given."""
    N, D, V, dt = _check_inputs(H, W, targets)
    dev = H.device
    lse = _vec(lse, N, dev, "lse")
    grad_loss = _vec(grad_loss, N, dev, "grad_loss")
    dH = _mat(dH, N, D, dev, "dH")
    dW = _mat(dW, V, D, dev, "dW")
    nbytes = flce_backward_workspace_bytes(N, D, V, dt)
    if nbytes == 0:
        raise FlceError(FLCE_ERR_UNSUPPORTED, "flce_backward_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rc = _lib.flce_backward(_ptr(H), _ptr(W), _ptr(targets), _ptr(lse), _ptr(grad_loss), N, D, V, dt,
                            _ptr(dH), _ptr(dW), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream_ptr(stream, dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_backward")
    return dH, dW


def forward(H, W, targets):
    """Convenience: (loss, lse) on the current stream with a library-managed workspace."""
    return flce_forward(H, W, targets)


def flce_forward_quant_workspace_bytes(N: int, D: int, V: int, bits: int, group: int) -> int:
    return int(_lib.flce_forward_quant_workspace_bytes(N, D, V, bits, group))


def _check_quant(H, codes, scales, biases, targets, bits, group):
    for name, t in (("H", H), ("codes", codes), ("scales", scales), ("biases", biases), ("targets", targets)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous torch.Tensor on a GPU device")
    if H.dtype != torch.bfloat16 or H.dim() != 2:
        raise ValueError("H must be a (N, D) bfloat16 tensor")
    N, D = H.shape
    V = codes.shape[0]
    if codes.dtype != torch.uint8 or codes.dim() != 2 or bits not in (4, 8) or \
            codes.shape[1] != (D if bits == 8 else D // 2):
        raise ValueError(f"codes must be uint8 of shape (V, {D if bits == 8 else D // 2}) for bits={bits}")
    if group <= 0 or D % group:
        raise ValueError(f"group must divide D={D}")
    for name, t in (("scales", scales), ("biases", biases)):
        if t.dtype != torch.float32 or t.shape != (V, D // group):
            raise ValueError(f"{name} must be float32 of shape ({V}, {D // group})")
    if targets.dtype != torch.int32 or targets.shape != (N,):
        raise ValueError("targets must be int32 of shape (N,)")
    return N, D, V


def flce_forward_quant(H, codes, scales, biases, targets, bits: int, group: int, workspace=None,
                       loss=None, lse=None, stream=None):
    """(loss, lse) for a quantised head: codes (V, D) uint8 at 8 bits or (V, D/2)
    at 4 bits (two per byte, low nibble first), scales and biases float32
    (V, D/group); see flce_forward_quant in include/flce.h for the format."""
    N, D, V = _check_quant(H, codes, scales, biases, targets, bits, group)
    dev = H.device
    loss = _out(loss, N, dev, "loss")
    lse = _out(lse, N, dev, "lse")
    nbytes = flce_forward_quant_workspace_bytes(N, D, V, bits, group)
    if N and nbytes == 0:
        raise FlceError(FLCE_ERR_UNSUPPORTED, "flce_forward_quant_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = _lib.flce_forward_quant(_ptr(H), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(targets), N, D, V,
                                 bits, group, _ptr(loss), _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward_quant")
    return loss, lse


def flce_backward_quant_workspace_bytes(N: int, D: int, V: int, bits: int, group: int) -> int:
    return int(_lib.flce_backward_quant_workspace_bytes(N, D, V, bits, group))


def flce_backward_quant(H, codes, scales, biases, targets, lse, grad_loss, bits: int, group: int,
                        workspace=None, dH=None, stream=None):
    """dH (float32) of sum_i grad_loss[i] * loss_i for the quantised head, which
    is frozen (no gradient); lse is flce_forward_quant's lse for the same inputs."""
    N, D, V = _check_quant(H, codes, scales, biases, targets, bits, group)
    dev = H.device
    lse = _vec(lse, N, dev, "lse")
    grad_loss = _vec(grad_loss, N, dev, "grad_loss")
    dH = _mat(dH, N, D, dev, "dH")
    if N == 0:
        return dH
    nbytes = flce_backward_quant_workspace_bytes(N, D, V, bits, group)
    if nbytes == 0:
        raise FlceError(FLCE_ERR_UNSUPPORTED, "flce_backward_quant_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rc = _lib.flce_backward_quant(_ptr(H), _ptr(codes), _ptr(scales), _ptr(biases), _ptr(targets), _ptr(lse),
                                  _ptr(grad_loss), N, D, V, bits, group, _ptr(dH), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_backward_quant")
    return dH


class LinearCrossEntropyQuant(torch.autograd.Function):
    """Per-token loss for a quantised head, differentiable in H only (the head
    is frozen): forward flce_forward_quant, backward flce_backward_quant with
    the saved lse."""

    @staticmethod
    def forward(ctx, H, codes, scales, biases, targets, bits, group):
        loss, lse = flce_forward_quant(H, codes, scales, biases, targets, bits, group)
        ctx.save_for_backward(H, codes, scales, biases, targets, lse)
        ctx.bits, ctx.group = bits, group
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        H, codes, scales, biases, targets, lse = ctx.saved_tensors
        dH = None
        if ctx.needs_input_grad[0]:
            g = grad_loss.to(torch.float32).contiguous()
            dH = flce_backward_quant(H, codes, scales, biases, targets, lse, g, ctx.bits, ctx.group)
        return dH, None, None, None, None, None, None


def linear_cross_entropy_quant(H, codes, scales, biases, targets, bits: int, group: int):
    """Per-token loss (float32, (N,)) with a quantised head in the format of
    flce_forward_quant; differentiable in H. Ignored positions (targets outside
    [0, V)) are handled as in linear_cross_entropy."""
    return LinearCrossEntropyQuant.apply(H, codes, scales, biases, targets, bits, group)


class LinearCrossEntropy(torch.autograd.Function):
    """Per-token loss with gradients for H and W: the forward runs flce_forward
    and keeps its lse; the backward hands the incoming per-token gradient to
    flce_backward, which regenerates the logits tile by tile, one vocabulary
    slice at a time, so dZ never exists beyond one slice (at most 1 GiB): the
    page's training path keeps the forward's log-sum-exp, not the logits, and
    runs a chunked backward. The float32 gradients are cast to the inputs'
    dtype by autograd itself."""

    @staticmethod
    def forward(ctx, H, W, targets):
        loss, lse = flce_forward(H, W, targets)
        ctx.save_for_backward(H, W, targets, lse)
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        H, W, targets, lse = ctx.saved_tensors
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1]):
            return None, None, None
        g = grad_loss.to(torch.float32).contiguous()
        dH, dW = flce_backward(H, W, targets, lse, g)
        return (dH if ctx.needs_input_grad[0] else None,
                dW if ctx.needs_input_grad[1] else None, None)


def linear_cross_entropy(H, W, targets):
    """loss_i = logsumexp(H_i W^T) - (H_i W^T)[y_i] per token (float32, shape
    (N,)), differentiable in H and W; reduce it (mean, weights) as needed.
    A target outside [0, V) (an ignored position) gives that row a NaN loss:
    select the valid rows before reducing, e.g. loss[y >= 0].mean(); the
    ignored rows then receive a zero upstream gradient and contribute nothing
    to dH or dW."""
    return LinearCrossEntropy.apply(H, W, targets)
