"""Autograd entry points with the semantics of the PyTorch module source
torch/nn/modules/linear_cross_entropy.py (the custom ops
_linear_cross_entropy_batch_chunked and ..._no_reduction with their autograd
registration) and of the torch.nn.LinearCrossEntropyOptions page.

Every number is computed by liblce.so; this module only resolves options into
the C descriptor, allocates outputs through PyTorch and hands pointers over.

* mean / sum: the forward forms the loss and every requested gradient in one
  pass; the backward multiplies the stored gradients by the incoming scalar
  gradient (lce_scale, on the device).  By default that happens in place and
  a second backward raises RuntimeError; allow_retain_graph=True scales into
  new buffers instead, at the cost of one gradient-sized allocation per
  backward.
* none: the forward returns the per-row loss and keeps the inputs; the
  backward recomputes the chunked pass with the per-row upstream gradient,
  so retain_graph always works and allow_retain_graph is ignored.
* Higher-order derivatives are not supported (the backward is
  once-differentiable).
* cross_entropy_inplace: softmax cross-entropy over given fp32 logits that
  overwrites the logits with the gradient (Liger-Kernel issue #343); the
  overwritten tensor is declared with mark_dirty.
"""
from __future__ import annotations

import dataclasses
import re

import torch
from torch.autograd.function import once_differentiable

from . import _binding as B
from .api import CrossEntropyInplace, LinearCrossEntropy, _stream

_LCE_DTYPE = {torch.float32: B.LCE_F32, torch.bfloat16: B.LCE_BF16, torch.float16: B.LCE_F16}


@dataclasses.dataclass(frozen=True)
class LinearCrossEntropyOptions:
    """The fields of torch.nn.LinearCrossEntropyOptions.

    chunking_method: "auto" (= "aspect_ratio"), "aspect_ratio",
    "aspect_ratio:N" or None (use batch_chunk_size; None there means one
    chunk).  acc_policy: "auto" (= "compact" on the GPU), "accurate" or
    "compact".  acc_dtype: None or torch.float32 (mixed precision for 16-bit
    inputs), or the input dtype itself (non-mixed: gradients accumulated chunk
    by chunk in the input dtype, as "compact")."""
    allow_retain_graph: bool = False
    batch_chunk_size: int | None = None
    chunking_method: str | None = "auto"
    acc_policy: str = "auto"
    acc_dtype: torch.dtype | None = None


_ASPECT = re.compile(r"^aspect_ratio(?::(\d+))?$")


def _resolve(opts: LinearCrossEntropyOptions, N: int, D: int, V: int, dtype) -> dict:
    """Options -> C descriptor fields (chunk_rows, chunk_divisor, acc_policy,
    acc_dtype)."""
    if opts.acc_policy not in ("auto", "accurate", "compact"):
        raise ValueError(f"unknown acc_policy {opts.acc_policy!r}")
    acc = torch.float32 if opts.acc_dtype is None else opts.acc_dtype
    # [LCE]: acc_dtype must equal the input dtype unless a 16-bit input
    # accumulates in float32 (mixed precision)
    if acc != torch.float32 and acc != dtype:
        raise RuntimeError(f"acc_dtype {acc} does not fit input dtype {dtype}")
    policy = "compact" if opts.acc_policy == "auto" else opts.acc_policy
    if acc == dtype and dtype != torch.float32:
        policy = "compact"           # non-mixed: every gradient buffer in the input dtype
    bcs = opts.batch_chunk_size
    if bcs is not None and (not isinstance(bcs, int) or bcs < 1):
        raise ValueError(f"batch_chunk_size must be a positive int, got {bcs!r}")
    method = opts.chunking_method
    if method is None:
        return {"chunk_rows": bcs if bcs is not None else B.LCE_CHUNK_ALL, "chunk_divisor": 1,
                "acc_policy": policy, "acc_dtype": acc}
    if method == "auto":
        if bcs is not None:          # the default method yields to an explicit size
            return {"chunk_rows": bcs, "chunk_divisor": 1, "acc_policy": policy,
                    "acc_dtype": acc}
        method = "aspect_ratio"
    m = _ASPECT.match(method)
    if m is None:
        raise ValueError(f"unknown chunking_method {method!r}")
    div = int(m.group(1) or 1)
    if div < 1:
        raise ValueError("aspect_ratio:N needs N >= 1")
    res = {"chunk_rows": B.LCE_CHUNK_ASPECT_RATIO, "chunk_divisor": div, "acc_policy": policy,
           "acc_dtype": acc}
    if bcs is not None:
        desc = B.lce_desc(N=N, D=D, V=V, ignore_index=-100, chunk_rows=B.LCE_CHUNK_ASPECT_RATIO,
                          dtype=_LCE_DTYPE[dtype], acc_dtype=B.LCE_F32, has_bias=0,
                          reduction=B.LCE_MEAN, acc_policy=B.LCE_COMPACT, flags=0,
                          chunk_divisor=div)
        h = B.lce_create(desc)
        try:
            rows, _ = B.lce_chunk_info(h)
        finally:
            B.lce_destroy(h)
        if rows != min(bcs, N):
            raise ValueError(f"batch_chunk_size={bcs} disagrees with chunking_method="
                             f"{opts.chunking_method!r} ({rows} rows)")
    return res


def _check_args(X, W, t, b, cw, reduction, label_smoothing):
    if reduction not in ("mean", "sum", "none"):
        # [LCE] _ChunkContext's validation: an unsupported reduction
        raise NotImplementedError(f"reduction={reduction!r} is not supported")
    if label_smoothing != 0.0:
        raise NotImplementedError("label_smoothing is not supported")
    if t.dtype != torch.int64:
        raise TypeError(f"target dtype must be torch.int64, got {t.dtype}")
    if X.dtype not in _LCE_DTYPE:
        raise NotImplementedError(f"input dtype {X.dtype} is not supported")
    if W.dtype != X.dtype or (b is not None and b.dtype != X.dtype):
        raise RuntimeError("input, linear_weight and linear_bias must share one dtype")
    if X.dim() < 1 or W.dim() != 2 or X.shape[-1] != W.shape[1]:
        raise RuntimeError(f"shape mismatch: input {tuple(X.shape)}, linear_weight "
                           f"{tuple(W.shape)}")
    if tuple(t.shape) != tuple(X.shape[:-1]):
        raise RuntimeError(f"target shape {tuple(t.shape)} does not match input "
                           f"{tuple(X.shape[:-1])}")
    if b is not None and tuple(b.shape) != (W.shape[0],):
        raise RuntimeError(f"expected bias shape {(W.shape[0],)}, got {tuple(b.shape)}")
    if cw is not None and (tuple(cw.shape) != (W.shape[0],) or not cw.is_floating_point()):
        raise RuntimeError(f"weight must be a float tensor of shape {(W.shape[0],)}")
    for name, x in (("input", X), ("linear_weight", W), ("target", t), ("linear_bias", b),
                    ("weight", cw)):
        if x is not None and x.device != X.device:
            raise RuntimeError(f"{name} is on {x.device}, input on {X.device}")


def _op(N, D, V, dtype, device, *, bias, reduction, ignore_index, cfg, gx, gw, gb):
    return LinearCrossEntropy(N, D, V, dtype, bias=bias, reduction=reduction,
                              ignore_index=ignore_index, chunk_rows=cfg["chunk_rows"],
                              chunk_divisor=cfg["chunk_divisor"], acc_policy=cfg["acc_policy"],
                              acc_dtype=cfg["acc_dtype"], grad_x=gx, grad_w=gw, grad_b=gb,
                              device=device)


class _ScalarLCE(torch.autograd.Function):
    """mean / sum: gradients formed in the forward, scaled in the backward."""

    @staticmethod
    def forward(ctx, X, W, t, b, cw, reduction, ignore_index, cfg, retain, grad_on):
        # needs_input_grad ignores no_grad mode: the caller passes grad_on
        need = [grad_on and bool(x) for x in ctx.needs_input_grad]
        gx, gw, gb = need[0], need[1], b is not None and need[3]
        N, D = X.shape
        op = _op(N, D, W.shape[0], X.dtype, X.device, bias=b is not None, reduction=reduction,
                 ignore_index=ignore_index, cfg=cfg, gx=gx, gw=gw, gb=gb)
        out = op(X, W, t, b, class_weight=cw)
        ctx.grads = [out.get("grad_X") if gx else None, out.get("grad_W") if gw else None,
                     out.get("grad_b") if gb else None]
        ctx.lce_dtype = _LCE_DTYPE[X.dtype]
        ctx.device = X.device
        ctx.allow_retain_graph = retain
        ctx.consumed = False
        # the op's output contract (its fake-tensor registration in [LCE]): a
        # scalar of the input dtype, rounded once from the fp32 loss
        return out["loss"].reshape(()).to(X.dtype)

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_loss):
        if ctx.consumed and not ctx.allow_retain_graph:
            raise RuntimeError(
                "linear_cross_entropy: the gradient buffers formed in the forward were already "
                "scaled in place by an earlier backward; pass allow_retain_graph=True to "
                "backward through this graph more than once")
        ctx.consumed = True
        g = grad_loss.detach().to(device=ctx.device, dtype=torch.float32).reshape(1).contiguous()
        res = []
        for buf in ctx.grads:
            if buf is None:
                res.append(None)
                continue
            dst = torch.empty_like(buf) if ctx.allow_retain_graph else buf
            B.lce_scale(buf.data_ptr(), dst.data_ptr(), ctx.lce_dtype, 1, buf.numel(),
                        g.data_ptr(), 0, _stream())
            res.append(dst)
        if not ctx.allow_retain_graph:
            ctx.grads = [None, None, None]
        return res[0], res[1], None, res[2], None, None, None, None, None, None


class _NoneLCE(torch.autograd.Function):
    """none: per-row loss; the backward recomputes with the upstream rows."""

    @staticmethod
    def forward(ctx, X, W, t, b, cw, ignore_index, cfg):
        N, D = X.shape
        op = _op(N, D, W.shape[0], X.dtype, X.device, bias=b is not None, reduction="none",
                 ignore_index=ignore_index, cfg=cfg, gx=False, gw=False, gb=False)
        out = op(X, W, t, b, class_weight=cw)
        ctx.save_for_backward(X, W, t, b, cw)
        ctx.ignore_index = ignore_index
        ctx.cfg = cfg
        return out["loss"].to(X.dtype)            # [LCE]: (N,) of the input dtype

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_rows):
        X, W, t, b, cw = ctx.saved_tensors
        need = ctx.needs_input_grad
        gx, gw, gb = bool(need[0]), bool(need[1]), b is not None and bool(need[3])
        if not (gx or gw or gb):
            return None, None, None, None, None, None, None
        N, D = X.shape
        op = _op(N, D, W.shape[0], X.dtype, X.device, bias=b is not None, reduction="none",
                 ignore_index=ctx.ignore_index, cfg=ctx.cfg, gx=gx, gw=gw, gb=gb)
        u = grad_rows.detach().to(device=X.device, dtype=torch.float32).contiguous()
        out = op(X, W, t, b, grad_output=u, class_weight=cw)
        return (out.get("grad_X") if gx else None, out.get("grad_W") if gw else None, None,
                out.get("grad_b") if gb else None, None, None, None)


def linear_cross_entropy(input, linear_weight, target, linear_bias=None, weight=None,
                         reduction: str = "mean", ignore_index: int = -100,
                         label_smoothing: float = 0.0,
                         options: LinearCrossEntropyOptions | None = None):
    """cross_entropy(input @ linear_weight.T + linear_bias, target) without
    the logits, differentiable in input, linear_weight and linear_bias.

    input (*, D) float32, bfloat16 or float16, linear_weight (V, D), target
    (*) int64, linear_bias (V,) or None, weight (V,) per-class weights or
    None.  Returns the loss in the input dtype (the module source's output
    contract: the fp32 loss rounded once): a scalar for mean / sum, the
    per-row loss of target's shape for none."""
    opts = options or LinearCrossEntropyOptions()
    _check_args(input, linear_weight, target, linear_bias, weight, reduction, label_smoothing)
    lead = tuple(target.shape)
    D = input.shape[-1]
    X = input.reshape(-1, D).contiguous()
    t = target.reshape(-1).contiguous()
    W = linear_weight.contiguous()
    b = None if linear_bias is None else linear_bias.contiguous()
    cw = None if weight is None else weight.detach().to(torch.float32).contiguous()
    cfg = _resolve(opts, X.shape[0], D, W.shape[0], X.dtype)
    if reduction == "none":
        return _NoneLCE.apply(X, W, t, b, cw, ignore_index, cfg).reshape(lead)
    return _ScalarLCE.apply(X, W, t, b, cw, reduction, ignore_index, cfg,
                            bool(opts.allow_retain_graph), torch.is_grad_enabled())


class _CEInplace(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, t, cw, reduction, ignore_index):
        op = CrossEntropyInplace(logits.shape[0], logits.shape[1], reduction=reduction,
                                 ignore_index=ignore_index, device=logits.device)
        loss, _ = op(logits, t, 1.0, cw)
        ctx.set_materialize_grads(False)   # no zero tensor for the unused logits output
        ctx.mark_dirty(logits)
        ctx.save_for_backward(logits)
        ctx.reduction = reduction
        return loss if reduction == "none" else loss.reshape(()), logits

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_loss, grad_logits):
        # The public wrapper drops the overwritten logits, so nothing flows
        # back through them.
        assert grad_logits is None
        (dl,) = ctx.saved_tensors
        if grad_loss is None:
            return None, None, None, None, None
        # the stored rows are the weighted softmax - onehot of each row: times
        # the scalar upstream gradient (mean / sum) or row n times u_n (none)
        g = torch.empty_like(dl)
        u = grad_loss.detach().to(device=dl.device, dtype=torch.float32).reshape(-1).contiguous()
        per_row = ctx.reduction == "none"
        B.lce_scale(dl.data_ptr(), g.data_ptr(), B.LCE_F32, dl.shape[0] if per_row else 1,
                    dl.shape[1] if per_row else dl.numel(), u.data_ptr(), 1 if per_row else 0,
                    _stream())
        return g, None, None, None, None


def cross_entropy_inplace(logits, target, weight=None, reduction: str = "mean",
                          ignore_index: int = -100):
    """Softmax cross-entropy over fp32 logits [N, V] that overwrites the logits
    with the gradient of the loss (declared to autograd with mark_dirty).
    Returns the loss; logits must not be a leaf that requires grad."""
    if reduction not in ("mean", "sum", "none"):
        # [LCE] _ChunkContext's validation: an unsupported reduction
        raise NotImplementedError(f"reduction={reduction!r} is not supported")
    if target.dtype != torch.int64:
        raise TypeError(f"target dtype must be torch.int64, got {target.dtype}")
    cw = None if weight is None else weight.detach().to(torch.float32).contiguous()
    loss, _ = _CEInplace.apply(logits, target.contiguous(), cw, reduction, ignore_index)
    return loss
