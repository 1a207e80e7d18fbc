"""torch-facing wrappers over the C ABI.

PyTorch supplies device memory (outputs and the workspace) and the stream
(torch's current stream); the computation itself runs entirely in liblce.so.
The argument checks mirror the pages' Python validation that a C pointer
cannot carry: the target dtype (int64, a TypeError on the pages) and the bias
shape (a RuntimeError on the pages). Per-class weights, when given, are one
float32 value per class on the problem's device.

Every tensor whose pointer reaches a kernel is checked on the host before
anything is enqueued: its device (the op's), its shape and its contiguity.
A host tensor or a short buffer would otherwise be read by the kernels out
of bounds.
"""
from __future__ import annotations

import torch

from . import _binding as B

_DTYPES = {torch.float32: B.LCE_F32, torch.bfloat16: B.LCE_BF16, torch.float16: B.LCE_F16}
_REDUCTIONS = {"mean": B.LCE_MEAN, "sum": B.LCE_SUM, "none": B.LCE_NONE}
_POLICIES = {"accurate": B.LCE_ACCURATE, "compact": B.LCE_COMPACT}


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_class_weight(w, V: int, device: torch.device) -> None:
    if w is not None and (w.dtype != torch.float32 or tuple(w.shape) != (V,)
                          or not w.is_contiguous() or w.device != device):
        raise RuntimeError(f"class_weight must be a contiguous float32 tensor of shape ({V},) "
                           f"on {device}")


def _check_tensor(name: str, x, shape: tuple, dtype, device: torch.device) -> None:
    """x must be a contiguous tensor of `shape` and `dtype` on `device`."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(x).__name__}")
    if x.device != device:
        raise RuntimeError(f"{name} is on {x.device}, expected {device}")
    if tuple(x.shape) != tuple(shape):
        raise RuntimeError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if x.dtype != dtype:
        raise RuntimeError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")


def _device(device) -> torch.device:
    d = torch.device(device)
    if d.type == "cuda" and d.index is None:
        d = torch.device("cuda", torch.cuda.current_device())
    return d


class LinearCrossEntropy:
    """A planned chunked linear-cross-entropy problem of fixed shape.

    Holds the C handle and a torch-allocated workspace; each call enqueues
    one lce_forward_backward on torch's current stream."""

    def __init__(self, N: int, D: int, V: int, dtype: torch.dtype, *, bias: bool = False,
                 reduction: str = "mean", ignore_index: int = -100, chunk_rows: int = 0,
                 acc_policy: str = "accurate", grad_x: bool = True, grad_w: bool = True,
                 grad_b: bool | None = None, argmax: bool = False, device="cuda",
                 chunk_divisor: int = 1, accumulate: bool = False, acc_dtype=None,
                 group_rows: int = 0):
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}")
        if reduction not in _REDUCTIONS:
            raise NotImplementedError(f"reduction={reduction!r} is not supported")
        # None / float32: mixed precision; the input dtype itself: non-mixed
        acc = torch.float32 if acc_dtype is None else acc_dtype
        if acc not in _DTYPES:
            raise TypeError(f"unsupported acc_dtype {acc}")
        grad_b = bias if grad_b is None else grad_b
        flags = ((B.LCE_GRAD_X if grad_x else 0) | (B.LCE_GRAD_W if grad_w else 0) |
                 (B.LCE_GRAD_B if grad_b else 0) | (B.LCE_ARGMAX if argmax else 0) |
                 (B.LCE_ACCUMULATE if accumulate else 0))
        self.accumulate = accumulate
        self.shape = (N, D, V)
        self.dtype = dtype
        self.bias = bias
        self.reduction = reduction
        self.flags = flags
        self.device = _device(device)
        self.desc = B.lce_desc(N=N, D=D, V=V, ignore_index=ignore_index, chunk_rows=chunk_rows,
                               dtype=_DTYPES[dtype], acc_dtype=_DTYPES[acc], has_bias=int(bias),
                               reduction=_REDUCTIONS[reduction],
                               acc_policy=_POLICIES[acc_policy], flags=flags,
                               chunk_divisor=chunk_divisor, group_rows=group_rows)
        self.handle = B.lce_create(self.desc)
        self.ws_bytes = B.lce_workspace_size(self.handle)
        self.chunk_rows, self.n_chunks = B.lce_chunk_info(self.handle)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8,
                                     device=self.device)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None:
            try:
                B.lce_destroy(h)
            except Exception:
                pass
            self.handle = None

    def make_outputs(self, grads: bool = True) -> dict:
        N, D, V = self.shape
        dev, dt = self.device, self.dtype
        out = {
            "loss": torch.empty(N if self.reduction == "none" else 1, dtype=torch.float32,
                                device=dev),
            "n_valid": torch.empty(1, dtype=torch.int64, device=dev),
            "n_bad": torch.empty(1, dtype=torch.int64, device=dev),
        }
        if grads and self.flags & B.LCE_GRAD_X:
            out["grad_X"] = torch.empty(N, D, dtype=dt, device=dev)
        if grads and self.flags & B.LCE_GRAD_W:
            out["grad_W"] = torch.empty(V, D, dtype=dt, device=dev)
        if grads and self.flags & B.LCE_GRAD_B:
            out["grad_b"] = torch.empty(V, dtype=dt, device=dev)
        if self.flags & B.LCE_ARGMAX:
            out["argmax"] = torch.empty(N, dtype=torch.int32, device=dev)
        return out

    def check_inputs(self, X, W, t, b=None, grad_output=None, class_weight=None) -> None:
        N, D, V = self.shape
        _check_class_weight(class_weight, V, self.device)
        if t.dtype != torch.int64:
            raise TypeError(f"target dtype must be torch.int64, got {t.dtype}")
        if b is not None and tuple(b.shape) != (V,):
            raise RuntimeError(f"expected bias shape {(V,)}, got {tuple(b.shape)}")
        if (b is not None) != self.bias:
            raise RuntimeError("bias presence differs from the planned problem")
        if tuple(X.shape) != (N, D) or tuple(W.shape) != (V, D) or tuple(t.shape) != (N,):
            raise RuntimeError(f"shape mismatch: X{tuple(X.shape)} W{tuple(W.shape)} "
                               f"t{tuple(t.shape)} vs planned N={N} D={D} V={V}")
        _check_tensor("X", X, (N, D), self.dtype, self.device)
        _check_tensor("W", W, (V, D), self.dtype, self.device)
        _check_tensor("target", t, (N,), torch.int64, self.device)
        if b is not None:
            _check_tensor("b", b, (V,), self.dtype, self.device)
        if grad_output is not None:
            _check_tensor("grad_output", grad_output, (N,), torch.float32, self.device)

    def check_outputs(self, out: dict, grads: bool = True) -> None:
        """Caller-supplied outputs: the requested gradients with their shapes."""
        N, D, V = self.shape
        want = (("grad_X", B.LCE_GRAD_X, (N, D)), ("grad_W", B.LCE_GRAD_W, (V, D)),
                ("grad_b", B.LCE_GRAD_B, (V,)))
        for name, flag, shape in want:
            if not grads or not self.flags & flag:
                continue
            g = out.get(name)
            if (g is None or tuple(g.shape) != shape or g.dtype != self.dtype
                    or not g.is_contiguous() or g.device != self.device):
                raise RuntimeError(f"out[{name!r}] must be a contiguous {self.dtype} tensor of "
                                   f"shape {shape} on {self.device}")
        for name, n, dt in (("loss", N if self.reduction == "none" else 1, torch.float32),
                            ("n_valid", 1, torch.int64), ("n_bad", 1, torch.int64),
                            ("argmax", N, torch.int32)):
            x = out.get(name)
            if x is not None and (x.numel() != n or x.dtype != dt or x.device != self.device
                                  or not x.is_contiguous()):
                raise RuntimeError(f"out[{name!r}] must hold {n} contiguous {dt} on "
                                   f"{self.device}")

    def make_io(self, X, W, t, b=None, *, out: dict, grad_output=None,
                grad_scale: float = 1.0, class_weight=None) -> B.lce_io:
        return B.lce_io(X=_ptr(X), W=_ptr(W), b=_ptr(b), targets=_ptr(t),
                        grad_output=_ptr(grad_output), loss=_ptr(out.get("loss")),
                        grad_X=_ptr(out.get("grad_X")), grad_W=_ptr(out.get("grad_W")),
                        grad_b=_ptr(out.get("grad_b")), argmax=_ptr(out.get("argmax")),
                        n_valid=_ptr(out.get("n_valid")), n_bad=_ptr(out.get("n_bad")),
                        grad_scale=grad_scale, reserved=0, class_weight=_ptr(class_weight))

    def run_io(self, io: B.lce_io) -> None:
        B.lce_forward_backward(self.handle, io, self.workspace.data_ptr(), self.ws_bytes,
                               _stream())

    def __call__(self, X, W, t, b=None, *, grad_output=None, grad_scale: float = 1.0,
                 class_weight=None, out: dict | None = None) -> dict:
        self.check_inputs(X, W, t, b, grad_output, class_weight)
        grads = self.reduction != "none" or grad_output is not None
        if out is None:
            if self.accumulate and grads:
                raise ValueError("accumulate adds into existing gradients: pass them in out=")
            out = self.make_outputs(grads)
        else:
            full = self.make_outputs(grads=False)   # loss, counts, argmax the caller left out
            full.update(out)
            out = full
            self.check_outputs(out, grads)
        io = self.make_io(X, W, t, b, out=out, grad_output=grad_output, grad_scale=grad_scale,
                          class_weight=class_weight)
        self.run_io(io)
        return out


def linear_cross_entropy(X, W, t, b=None, *, reduction: str = "mean", ignore_index: int = -100,
                         chunk_rows: int = 0, acc_policy: str = "accurate",
                         grad_output=None, grad_scale: float = 1.0, argmax: bool = False,
                         grad_x: bool = True, grad_w: bool = True,
                         grad_b: bool | None = None, class_weight=None,
                         group_rows: int = 0) -> dict:
    """One-shot chunked forward+backward; returns loss, gradients, counts."""
    N, D = X.shape
    V = W.shape[0]
    op = LinearCrossEntropy(N, D, V, X.dtype, bias=b is not None, reduction=reduction,
                            ignore_index=ignore_index, chunk_rows=chunk_rows,
                            acc_policy=acc_policy, grad_x=grad_x, grad_w=grad_w,
                            grad_b=grad_b, argmax=argmax, device=X.device,
                            group_rows=group_rows)
    return op(X, W, t, b, grad_output=grad_output, grad_scale=grad_scale,
              class_weight=class_weight)


class CrossEntropyInplace:
    """Standalone softmax cross-entropy over fp32 logits [N, V]; the logits are
    overwritten with the gradient."""

    def __init__(self, N: int, V: int, *, reduction: str = "mean", ignore_index: int = -100,
                 device="cuda"):
        if reduction not in _REDUCTIONS:
            raise NotImplementedError(f"reduction={reduction!r} is not supported")
        self.N, self.V = N, V
        self.reduction = reduction
        self.ignore_index = ignore_index
        self.device = _device(device)
        self.ws_bytes = B.lce_ce_workspace_size(N, V)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8,
                                     device=self.device)
        self.loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32,
                                device=self.device)
        self.n_valid = torch.empty(1, dtype=torch.int64, device=self.device)

    def __call__(self, logits: torch.Tensor, t: torch.Tensor, grad_scale: float = 1.0,
                 class_weight=None):
        _check_class_weight(class_weight, self.V, self.device)
        if t.dtype != torch.int64:
            raise TypeError(f"target dtype must be torch.int64, got {t.dtype}")
        _check_tensor("logits", logits, (self.N, self.V), torch.float32, self.device)
        _check_tensor("target", t, (self.N,), torch.int64, self.device)
        B.lce_ce_inplace(logits.data_ptr(), t.data_ptr(), _ptr(class_weight), self.N, self.V,
                         self.ignore_index,
                         _REDUCTIONS[self.reduction], grad_scale, self.loss.data_ptr(),
                         self.n_valid.data_ptr(), self.workspace.data_ptr(), self.ws_bytes,
                         _stream())
        return self.loss, self.n_valid


def cross_entropy_inplace(logits, t, *, reduction: str = "mean", ignore_index: int = -100,
                          grad_scale: float = 1.0, class_weight=None):
    op = CrossEntropyInplace(logits.shape[0], logits.shape[1], reduction=reduction,
                             ignore_index=ignore_index, device=logits.device)
    return op(logits, t, grad_scale, class_weight)
