"""Fused output projection + sparse top-K KL loss for AMD MI355X.

A thin ctypes binding over ``libfkl.so`` (C ABI declared in ``include/fkl.h``).
Every step of the loss runs in the library's HIP kernels; this module only
checks tensors, allocates outputs and workspace through torch, and passes
device pointers and torch's current stream. There is no fallback: if the
library is missing, every call raises.

The method (blog post on the page "Efficient Offline Top-K Logits and Fused
Chunked KL Loss Enable Scalable LLM Distillation", section "Two systems
changes"): the student's output projection is fused into a KL loss against
the teacher's cached top-K logits; the logits are formed one chunk at a time
and never stored, and backward forms them again.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "FklError",
    "lib",
    "library_path",
    "Shape",
    "workspace_size",
    "forward",
    "forward_static",
    "STATIC_SCRATCH_BYTES",
    "backward",
    "validate_teacher",
    "validate_terms",
    "plan_info",
    "PlanInfo",
    "FusedKLLoss",
    "Terms",
    "ACCUMULATE_GRAD_W",
    "ACCUMULATE_GRAD_H",
    "SKIP_GRAD_W",
    "SKIP_GRAD_H",
    "GRAD_H_BF16",
    "TopkShape",
    "topk_workspace_size",
    "topk",
    "trace_enable",
    "trace_read",
    "EXPORTED_SYMBOLS",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfkl.so"
_lib = None

EXPORTED_SYMBOLS = (
    "fkl_workspace_size",
    "fkl_forward",
    "fkl_forward_static",
    "fkl_backward",
    "fkl_validate_teacher",
    "fkl_validate_terms",
    "fkl_plan_info",
    "fkl_topk_workspace_size",
    "fkl_topk",
    "fkl_trace_enable",
    "fkl_trace_read",
    "fkl_status_string",
    "fkl_last_error",
    "fkl_version",
)


class FklError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfkl status {status}: {message}")
        self.status = status


class KernelStat(ctypes.Structure):
    """Mirror of ``fkl_kernel_stat``."""

    _fields_ = [
        ("name", ctypes.c_char * 32),
        ("launches", ctypes.c_int64),
        ("total_ms", ctypes.c_double),
        ("min_ms", ctypes.c_double),
        ("max_ms", ctypes.c_double),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
    ]


class Shape(ctypes.Structure):
    """Mirror of ``fkl_shape``."""

    _fields_ = [
        ("N", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("K", ctypes.c_int32),
        ("T", ctypes.c_float),
        ("chunk", ctypes.c_int32),
        ("vslab", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class Terms(ctypes.Structure):
    """Mirror of ``fkl_terms``."""

    _fields_ = [
        ("row_weight", ctypes.c_void_p),
        ("label", ctypes.c_void_p),
        ("label_weight", ctypes.c_float),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``fkl_plan``."""

    _fields_ = [
        ("fwd_rows", ctypes.c_int64),
        ("bwd_rows", ctypes.c_int64),
        ("vslab", ctypes.c_int64),
        ("fwd_passes", ctypes.c_int64),
        ("bwd_passes", ctypes.c_int64),
        ("slabs", ctypes.c_int64),
        ("fwd_bytes", ctypes.c_size_t),
        ("bwd_bytes", ctypes.c_size_t),
    ]


class TopkShape(ctypes.Structure):
    """Mirror of ``fkl_topk_shape``."""

    _fields_ = [
        ("N", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("K", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


TOPK_DIRECT = 0x1
TOPK_MATERIALIZE = 0x2


def library_path() -> str:
    return os.environ.get("FKL_LIBRARY", os.path.join(_PKG_DIR, _LIB_NAME))


def lib() -> ctypes.CDLL:
    """Load libfkl.so (built by ``python -m output_projection_kl_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FklError(-1, f"{path} is missing; build it with `python -m output_projection_kl_amd.build`")
    L = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    shp = ctypes.POINTER(Shape)
    L.fkl_workspace_size.argtypes = [shp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.fkl_forward.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fkl_forward_static.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.fkl_backward.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.fkl_validate_teacher.argtypes = [shp, vp, vp, vp, vp]
    L.fkl_validate_terms.argtypes = [shp, ctypes.POINTER(Terms), vp, vp]
    L.fkl_plan_info.argtypes = [shp, ctypes.POINTER(PlanInfo)]
    tshp = ctypes.POINTER(TopkShape)
    L.fkl_topk_workspace_size.argtypes = [tshp, ctypes.POINTER(sz)]
    L.fkl_topk.argtypes = [tshp, vp, vp, vp, vp, vp, sz, vp]
    L.fkl_trace_enable.argtypes = [ctypes.c_int]
    L.fkl_trace_read.argtypes = [ctypes.POINTER(KernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    for f in ("fkl_workspace_size", "fkl_forward", "fkl_forward_static", "fkl_backward", "fkl_validate_teacher", "fkl_validate_terms",
              "fkl_plan_info", "fkl_version",
              "fkl_topk_workspace_size", "fkl_topk", "fkl_trace_enable", "fkl_trace_read"):
        getattr(L, f).restype = ctypes.c_int
    L.fkl_status_string.argtypes = [ctypes.c_int]
    L.fkl_status_string.restype = ctypes.c_char_p
    L.fkl_last_error.argtypes = []
    L.fkl_last_error.restype = ctypes.c_char_p
    L.fkl_version.argtypes = []
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise FklError(status, f"{L.fkl_status_string(status).decode()}: {L.fkl_last_error().decode()}")


# Backward options (fkl_shape.flags; see include/fkl.h).
ACCUMULATE_GRAD_W = 0x1
ACCUMULATE_GRAD_H = 0x2
SKIP_GRAD_W = 0x4
SKIP_GRAD_H = 0x8
GRAD_H_BF16 = 0x10


def make_shape(N, d, V, K, T=1.0, chunk=0, vslab=0, flags=0) -> Shape:
    return Shape(int(N), int(d), int(V), int(K), float(T), int(chunk), int(vslab), int(flags))


def workspace_size(N, d, V, K, T=1.0, chunk=0, vslab=0, flags=0):
    """(forward_bytes, backward_bytes) of workspace for this shape."""
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    s = make_shape(N, d, V, K, T, chunk, vslab, flags)
    _check(lib().fkl_workspace_size(ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def plan_info(N, d, V, K, T=1.0, chunk=0, vslab=0, flags=0) -> dict:
    """How the library runs this shape: rows per forward / backward pass, the
    backward slab, pass and slab counts, workspace bytes (host only)."""
    s = make_shape(N, d, V, K, T, chunk, vslab, flags)
    p = PlanInfo()
    _check(lib().fkl_plan_info(ctypes.byref(s), ctypes.byref(p)))
    return {f: int(getattr(p, f)) for f, _ in PlanInfo._fields_}


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device):
    """Makes `device` current for a library call (its kernels run on the current device)."""
    return _torch().cuda.device(device)


def _need(t, name, dtype, shape, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, like h; got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _inputs(h, W, t_idx, t_logit, mask):
    torch = _torch()
    if h.dim() != 2 or W.dim() != 2 or t_idx.dim() != 2:
        raise ValueError("h, W and t_idx must be 2-D")
    N, d = h.shape
    V = W.shape[0]
    K = t_idx.shape[1]
    _need(h, "h", torch.bfloat16, (N, d))
    dev = h.device
    _need(W, "W", torch.bfloat16, (V, d), dev)
    _need(t_idx, "t_idx", torch.int32, (N, K), dev)
    _need(t_logit, "t_logit", torch.float32, (N, K), dev)
    if mask is not None:
        _need(mask, "mask", torch.uint8, (N,), dev)
    return N, d, V, K


def _terms(N, V, row_weight, label, label_weight, device=None):
    """ctypes fkl_terms for the optional loss terms, or None for the plain loss."""
    torch = _torch()
    if row_weight is None and label is None:
        return None
    if row_weight is not None:
        _need(row_weight, "row_weight", torch.float32, (N,), device)
    if label is not None:
        _need(label, "label", torch.int32, (N,), device)
    return Terms(_ptr(row_weight), _ptr(label), float(label_weight))


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        if _nbytes(workspace) < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def forward(h, W, t_idx, t_logit, T: float = 1.0, mask=None, chunk: int = 0, vslab: int = 0,
            workspace=None, return_row_kl: bool = False, loss=None, row_lse=None, row_kl=None,
            row_weight=None, label=None, label_weight: float = 0.0):
    """Fused forward. Returns (loss [1], row_lse [N]) or (loss, row_lse, row_kl).

    Output tensors may be passed in to be overwritten (no allocation).
    row_weight (fp32 [N]), label (int32 [N]) and label_weight select the loss
    variants of include/fkl.h (weighted mean; KL mixed with hard-label CE)."""
    torch = _torch()
    N, d, V, K = _inputs(h, W, t_idx, t_logit, mask)
    terms = _terms(N, V, row_weight, label, label_weight, h.device)
    s = make_shape(N, d, V, K, T, chunk, vslab)
    fb, _ = workspace_size(N, d, V, K, T, chunk, vslab)
    ws = _workspace(fb, h.device, workspace)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=h.device)
    _need(loss, "loss", torch.float32, (1,), h.device)
    if row_lse is None:
        row_lse = torch.empty(N, dtype=torch.float32, device=h.device)
    _need(row_lse, "row_lse", torch.float32, (N,), h.device)
    if return_row_kl and row_kl is None:
        row_kl = torch.empty(N, dtype=torch.float32, device=h.device)
    if row_kl is not None:
        _need(row_kl, "row_kl", torch.float32, (N,), h.device)
        return_row_kl = True
    with _on(h.device):
        _check(lib().fkl_forward(ctypes.byref(s), _ptr(h), _ptr(W), _ptr(t_idx), _ptr(t_logit), _ptr(mask),
                                 None if terms is None else ctypes.byref(terms), _ptr(loss), _ptr(row_lse),
                                 _ptr(row_kl), _ptr(ws), ctypes.c_size_t(_nbytes(ws)), _stream(h.device)))
    return (loss, row_lse, row_kl) if return_row_kl else (loss, row_lse)


STATIC_SCRATCH_BYTES = 32 << 20  # FKL_STATIC_SCRATCH_BYTES


def forward_static(h, W, t_idx, t_logit, T: float = 1.0, mask=None, chunk: int = 0, vslab: int = 0,
                   loss=None, row_lse=None, row_kl=None, return_row_kl: bool = False, row_weight=None,
                   label=None, label_weight: float = 0.0):
    """fkl_forward_static: the forward with the library's static device scratch
    instead of a workspace (no allocation inside the library; pass the output
    tensors to avoid allocating them here too). Same results as forward(), up
    to fp32 summation order where the default slab's forward passes do not fit
    the scratch and the library takes 8192-row passes instead."""
    torch = _torch()
    N, d, V, K = _inputs(h, W, t_idx, t_logit, mask)
    terms = _terms(N, V, row_weight, label, label_weight, h.device)
    s = make_shape(N, d, V, K, T, chunk, vslab)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=h.device)
    _need(loss, "loss", torch.float32, (1,), h.device)
    if row_lse is None:
        row_lse = torch.empty(N, dtype=torch.float32, device=h.device)
    _need(row_lse, "row_lse", torch.float32, (N,), h.device)
    if return_row_kl and row_kl is None:
        row_kl = torch.empty(N, dtype=torch.float32, device=h.device)
    if row_kl is not None:
        _need(row_kl, "row_kl", torch.float32, (N,), h.device)
        return_row_kl = True
    with _on(h.device):
        _check(lib().fkl_forward_static(ctypes.byref(s), _ptr(h), _ptr(W), _ptr(t_idx), _ptr(t_logit), _ptr(mask),
                                        None if terms is None else ctypes.byref(terms), _ptr(loss), _ptr(row_lse),
                                        _ptr(row_kl), _stream(h.device)))
    return (loss, row_lse, row_kl) if return_row_kl else (loss, row_lse)


def backward(h, W, t_idx, t_logit, row_lse, T: float = 1.0, mask=None, grad_loss=None, chunk: int = 0,
             vslab: int = 0, workspace=None, grad_h=None, grad_W=None, need_grad_h: bool = True,
             need_grad_W: bool = True, accumulate_grad_h: bool = False, accumulate_grad_W: bool = False,
             grad_h_dtype=None, row_weight=None, label=None, label_weight: float = 0.0):
    """Fused backward with recomputation. Returns (grad_h [N, d], grad_W fp32 [V, d]); a
    gradient that is not needed comes back as None. grad_h is fp32, or bf16 when
    grad_h_dtype is torch.bfloat16 (or a bf16 grad_h is passed). With accumulate_*,
    the passed tensor is added to instead of overwritten."""
    torch = _torch()
    N, d, V, K = _inputs(h, W, t_idx, t_logit, mask)
    _need(row_lse, "row_lse", torch.float32, (N,), h.device)
    if grad_loss is not None:
        _need(grad_loss, "grad_loss", torch.float32, (1,), h.device)
    terms = _terms(N, V, row_weight, label, label_weight, h.device)
    if grad_h_dtype is None:
        grad_h_dtype = grad_h.dtype if grad_h is not None else torch.float32
    if grad_h_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("grad_h must be float32 or bfloat16")
    flags = ((0 if need_grad_h else SKIP_GRAD_H) | (0 if need_grad_W else SKIP_GRAD_W) |
             (ACCUMULATE_GRAD_H if accumulate_grad_h else 0) | (ACCUMULATE_GRAD_W if accumulate_grad_W else 0) |
             (GRAD_H_BF16 if grad_h_dtype == torch.bfloat16 else 0))
    if (accumulate_grad_h and need_grad_h and grad_h is None) or (accumulate_grad_W and need_grad_W and grad_W is None):
        raise ValueError("accumulating needs the tensor to accumulate into")
    s = make_shape(N, d, V, K, T, chunk, vslab, flags)
    _, bb = workspace_size(N, d, V, K, T, chunk, vslab, flags)
    ws = _workspace(bb, h.device, workspace)
    if not need_grad_h:
        grad_h = None
    elif grad_h is None:
        grad_h = torch.empty((N, d), dtype=grad_h_dtype, device=h.device)
    else:
        _need(grad_h, "grad_h", grad_h_dtype, (N, d), h.device)
    if not need_grad_W:
        grad_W = None
    elif grad_W is None:
        grad_W = torch.empty((V, d), dtype=torch.float32, device=h.device)
    else:
        _need(grad_W, "grad_W", torch.float32, (V, d), h.device)
    with _on(h.device):
        _check(lib().fkl_backward(ctypes.byref(s), _ptr(h), _ptr(W), _ptr(t_idx), _ptr(t_logit), _ptr(mask),
                                  None if terms is None else ctypes.byref(terms), _ptr(row_lse), _ptr(grad_loss),
                                  _ptr(grad_h), _ptr(grad_W), _ptr(ws), ctypes.c_size_t(_nbytes(ws)),
                                  _stream(h.device)))
    return grad_h, grad_W


class FusedKLLoss:
    """Autograd entry: ``FusedKLLoss.apply(h, W, t_idx, t_logit, T=1.0, mask=None, chunk=0)``
    returns the scalar loss; its backward runs fkl_backward, reading the upstream
    gradient on the device (no host synchronisation), returns grad_h in h's dtype
    and grad_W in fp32 (autograd casts it to W's dtype), and skips whichever of
    the two is not required."""

    _fn = None

    @classmethod
    def apply(cls, h, W, t_idx, t_logit, T: float = 1.0, mask=None, chunk: int = 0, row_weight=None,
              label=None, label_weight: float = 0.0):
        if cls._fn is None:
            torch = _torch()

            class _Fn(torch.autograd.Function):
                @staticmethod
                def forward(ctx, h, W, t_idx, t_logit, T, mask, chunk, row_weight, label, label_weight):
                    loss, lse = forward(h, W, t_idx, t_logit, T=T, mask=mask, chunk=chunk, row_weight=row_weight,
                                        label=label, label_weight=label_weight)
                    ctx.save_for_backward(h, W, t_idx, t_logit, lse, mask, row_weight, label)
                    ctx.T, ctx.chunk, ctx.label_weight = T, chunk, label_weight
                    return loss.reshape(())

                @staticmethod
                def backward(ctx, g):
                    h, W, t_idx, t_logit, lse, mask, row_weight, label = ctx.saved_tensors
                    need_h, need_W = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
                    if not (need_h or need_W):
                        return (None,) * 10
                    gl = g.detach().reshape(1).to(torch.float32).contiguous()
                    gh, gW = backward(h, W, t_idx, t_logit, lse, T=ctx.T, mask=mask, grad_loss=gl,
                                      chunk=ctx.chunk, need_grad_h=need_h, need_grad_W=need_W,
                                      grad_h_dtype=h.dtype if h.dtype == torch.bfloat16 else torch.float32,
                                      row_weight=row_weight, label=label, label_weight=ctx.label_weight)
                    return gh, gW, None, None, None, None, None, None, None, None

            cls._fn = _Fn
        return cls._fn.apply(h, W, t_idx, t_logit, T, mask, chunk, row_weight, label, label_weight)


def validate_teacher(t_idx, t_logit, V: int) -> int:
    """Number of teacher rows with an index outside [0, V), a repeated index, or a non-finite logit."""
    torch = _torch()
    N, K = t_idx.shape
    _need(t_idx, "t_idx", torch.int32, (N, K))
    _need(t_logit, "t_logit", torch.float32, (N, K), t_idx.device)
    s = make_shape(N, 8, V, K, 1.0)
    bad = torch.empty(1, dtype=torch.int32, device=t_idx.device)
    with _on(t_idx.device):
        _check(lib().fkl_validate_teacher(ctypes.byref(s), _ptr(t_idx), _ptr(t_logit), _ptr(bad),
                                          _stream(t_idx.device)))
    return int(bad.item())


def validate_terms(N: int, V: int, row_weight=None, label=None, label_weight: float = 0.0) -> int:
    """Number of rows whose hard label lies outside [0, V) or whose weight is not finite."""
    torch = _torch()
    ref = row_weight if row_weight is not None else label
    if ref is None:
        return 0
    terms = _terms(N, V, row_weight, label, label_weight, ref.device)
    s = make_shape(N, 8, V, 1, 1.0)
    bad = torch.empty(1, dtype=torch.int32, device=ref.device)
    with _on(ref.device):
        _check(lib().fkl_validate_terms(ctypes.byref(s), ctypes.byref(terms), _ptr(bad), _stream(ref.device)))
    return int(bad.item())


def topk_workspace_size(N, d, V, K, chunk=0, flags=0) -> int:
    """Workspace bytes of topk() for this shape."""
    s = TopkShape(N, d, V, K, chunk, flags)
    b = ctypes.c_size_t(0)
    _check(lib().fkl_topk_workspace_size(ctypes.byref(s), ctypes.byref(b)))
    return b.value


def topk(h, W, K: int, chunk: int = 0, workspace=None, t_idx=None, t_logit=None, direct: bool = False,
         materialize: bool = False):
    """Offline teacher cache: per row of h (bf16 [N,d]), the K largest logits of
    h W^T (W bf16 [V,d]), descending, ties by the lower index. By default the
    fused route (logits filtered against a per-row threshold as they are formed);
    materialize=True forms each block of rows' logits and selects there from a
    sampled threshold, direct=True does so over every whole row (same result on
    every route). Returns (t_idx int32 [N,K], t_logit fp32 [N,K])."""
    torch = _torch()
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h and W must be 2-D")
    N, d = h.shape
    V = W.shape[0]
    _need(h, "h", torch.bfloat16, (N, d))
    _need(W, "W", torch.bfloat16, (V, d), h.device)
    s = TopkShape(N, d, V, K, chunk, (TOPK_DIRECT if direct else 0) | (TOPK_MATERIALIZE if materialize else 0))
    b = ctypes.c_size_t(0)
    _check(lib().fkl_topk_workspace_size(ctypes.byref(s), ctypes.byref(b)))
    ws = _workspace(b.value, h.device, workspace)
    if t_idx is None:
        t_idx = torch.empty((N, K), dtype=torch.int32, device=h.device)
    _need(t_idx, "t_idx", torch.int32, (N, K), h.device)
    if t_logit is None:
        t_logit = torch.empty((N, K), dtype=torch.float32, device=h.device)
    _need(t_logit, "t_logit", torch.float32, (N, K), h.device)
    with _on(h.device):
        _check(lib().fkl_topk(ctypes.byref(s), _ptr(h), _ptr(W), _ptr(t_idx), _ptr(t_logit), _ptr(ws),
                              ctypes.c_size_t(_nbytes(ws)), _stream(h.device)))
    return t_idx, t_logit


def trace_enable(on: bool = True) -> None:
    """Switch the library's per-kernel event timing on or off (process-wide)."""
    _check(lib().fkl_trace_enable(1 if on else 0))


def trace_read() -> list:
    """Per-kernel timing recorded since the last read (waits for the events)."""
    cap = 64
    buf = (KernelStat * cap)()
    n = ctypes.c_int(0)
    _check(lib().fkl_trace_read(buf, cap, ctypes.byref(n)))
    out = []
    for i in range(min(n.value, cap)):
        k = buf[i]
        out.append(dict(name=k.name.decode(), launches=int(k.launches), total_ms=k.total_ms,
                        min_ms=k.min_ms, max_ms=k.max_ms, flops=k.flops, bytes=k.bytes))
    return out
