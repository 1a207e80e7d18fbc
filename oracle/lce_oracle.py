"""fp64 CPU oracle for chunked fused linear-cross-entropy (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP path.

It computes the plain, unchunked definition of what the chunked method
reaches (chunking over batch rows and fusing the passes only reorder the same
sums), in IEEE binary64, with numpy's matmul as the only library primitive.
Inputs are upcast exactly from their stored float32 / bf16 values.

Sources (the pages this follows):
  [LCE]  PyTorch module source ``torch/nn/modules/linear_cross_entropy.py``
         (batch-chunked linear cross-entropy: ``_ChunkContext``,
         ``_linear_cross_entropy_batch_chunked_accumulator`` and the custom
         ops built on it).
  [OPT]  ``torch.nn.LinearCrossEntropyOptions`` documentation page.
  [LIG]  Liger-Kernel issue #343, "cross entropy kernel: inplace modification
         of input".
  [NJT]  PyTorch commit "Fix NJT linear_backward() memory usage".

Notation: X[N,D] inputs, W[V,D] output-head weight, b[V] bias, t[N] int64
targets, z = X W^T + b the logits, P = softmax(z) by rows, Y = onehot(t),
g[N] the per-row weight (the negation of [LCE]'s ``neg_weight_target``), and
dL = g (P - Y) the gradient of the loss with respect to the logits.

Readings where the pages are silent (every one is listed in the design notes):
  * targets outside [0, V) that are not ignore_index ("bad" rows) are counted
    in n_bad and treated like ignored rows (loss 0, gradient 0, excluded from
    the mean's denominator); the pages would fault on the gather;
  * argmax breaks ties toward the lowest class index;
  * the loss is returned as float64 here (float32 on the device).

Pins: every function below is pinned by the CPU test suite against closed
forms, finite differences, invariants or an independent library routine; no
function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

REDUCTIONS = ("mean", "sum", "none")


# --------------------------------------------------------------------------
# Step 1: which rows count.  [LCE] ``_ChunkContext._mask`` marks rows whose
# target equals ignore_index; ``corrected_target`` replaces those targets by 0
# when ignore_index lies outside [0, V) so that gathers stay in range.
# --------------------------------------------------------------------------
def target_masks(t: np.ndarray, V: int, ignore_index: int):
    """Return (valid, bad, n_valid, n_bad) for int64 targets t.

    A row is ignored when t == ignore_index (checked before any correction,
    so an ignore_index inside [0, V) still ignores its rows)."""
    t = np.asarray(t, dtype=np.int64)
    ignored = t == ignore_index
    bad = (~ignored) & ((t < 0) | (t >= V))
    valid = (~ignored) & (~bad)
    return valid, bad, int(valid.sum()), int(bad.sum())


def corrected_targets(t: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Targets with every non-valid row replaced by class 0 ([LCE]
    ``corrected_target``; extended to bad rows by the reading above)."""
    return np.where(valid, np.asarray(t, dtype=np.int64), 0)


# --------------------------------------------------------------------------
# Step 2: per-row weights.  [LCE] ``_ChunkContext.neg_weight_target``: an
# unmasked row weighs weight[target] with per-class weights (1 without them),
# a masked row 0; "mean" divides by d = sum of the unmasked row weights and
# uses NaN as the divisor when d == 0, "sum" negates, and the reduction='none'
# backward folds the per-row upstream gradient in.  g below is the negation of
# that tensor, so dL = g (P - Y).
# --------------------------------------------------------------------------
def class_row_weights(valid: np.ndarray, tc: np.ndarray,
                      class_weight: np.ndarray | None = None) -> np.ndarray:
    """w[N] in float64: class_weight[t_n] (1 without class weights) on valid
    rows, 0 elsewhere."""
    if class_weight is None:
        return valid.astype(np.float64)
    cw = np.asarray(class_weight, np.float64)
    return np.where(valid, cw[tc], 0.0)


def row_weights(valid: np.ndarray, reduction: str, grad_scale: float = 1.0,
                upstream: np.ndarray | None = None, *, tc: np.ndarray | None = None,
                class_weight: np.ndarray | None = None) -> np.ndarray:
    """g[N] in float64, with w = class_row_weights(valid, tc, class_weight):

    mean: grad_scale * w / sum(w); NaN on every row when sum(w) == 0 (the
          pages divide by NaN there).
    sum:  grad_scale * w.
    none: upstream[n] * w (the backward of the per-row loss)."""
    if reduction not in REDUCTIONS:
        raise ValueError(reduction)
    w = class_row_weights(valid, tc, class_weight)
    if reduction == "mean":
        d = w.sum()
        return w * grad_scale / (d if d != 0 else np.nan)
    if reduction == "sum":
        return w * grad_scale
    if upstream is None:
        return w
    return w * np.asarray(upstream, dtype=np.float64)


# --------------------------------------------------------------------------
# Step 3: logits.  [LCE] main loop: ``ctx.mm(input, linear_weight.T)`` then
# ``logits.add_(linear_bias)``.
# --------------------------------------------------------------------------
def logits(X: np.ndarray, W: np.ndarray, b: np.ndarray | None) -> np.ndarray:
    z = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
    if b is not None:
        z = z + np.asarray(b, np.float64)[None, :]
    return z


# --------------------------------------------------------------------------
# Step 4: row-stable log-sum-exp.  [LCE] main loop: subtract the row max
# ("softmax stability"), exponentiate in place, sum in the accumulation dtype
# (``sumexp_``), take the log.
# --------------------------------------------------------------------------
def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    if z.shape[1] == 0:
        return np.full(z.shape[0], -np.inf)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


# --------------------------------------------------------------------------
# Step 5: per-row loss.  [LCE] loss-only branch for reduction='none' ("read
# the target logit before sumexp_"): loss_n = log(denominator) - shifted
# target logit, times the unsigned row weight; the scalar reductions
# accumulate the same terms ("output +=" / "output -=").
# --------------------------------------------------------------------------
def row_losses(z: np.ndarray, lse: np.ndarray, tc: np.ndarray,
               valid: np.ndarray, w: np.ndarray | None = None) -> np.ndarray:
    """w[n] (lse_n - z[n, t_n]) on valid rows, 0 elsewhere; w = 1 when None."""
    n = np.arange(z.shape[0])
    zt = z[n, tc] if z.shape[0] else np.zeros(0)
    loss = np.where(valid, lse - zt, 0.0)
    return loss if w is None else w * loss


def reduce_loss(loss_rows: np.ndarray, denom, reduction: str):
    """mean: sum / denom, denom the sum of the unmasked row weights (the
    count n_valid without class weights); NaN when denom == 0, including
    N == 0, as the pages fill the output with NaN for an empty mean.  sum:
    the sum; none: the per-row vector."""
    if reduction == "none":
        return loss_rows
    s = float(np.sum(loss_rows))
    if reduction == "sum":
        return s
    return s / denom if denom else float("nan")


# --------------------------------------------------------------------------
# Step 6: the logits gradient.  [LCE] main loop: the logits become
# softmax * w in place (``logits *= weight_chunk / softmax_denom``) and the
# one-hot part enters as ``index_select`` / ``index_add_`` corrections; in
# total dL[n, j] = g_n (P[n, j] - [j == t_n]).
# --------------------------------------------------------------------------
def dlogits(z: np.ndarray, lse: np.ndarray, tc: np.ndarray,
            g: np.ndarray) -> np.ndarray:
    P = np.exp(z - lse[:, None])
    Y = np.zeros_like(P)
    if z.shape[0]:
        Y[np.arange(z.shape[0]), tc] = 1.0
    return g[:, None] * (P - Y)


# --------------------------------------------------------------------------
# Step 7: the three gradients of the linear layer.  [LCE] input-grad
# ``addmm``, weight-grad ``mm``/``addmm_`` and bias-grad ``sum`` branches;
# [NJT] ``linear_backward``: ds = grad W, dw = grad^T input with leading dims
# folded to 2-D, db = sum over rows.
# --------------------------------------------------------------------------
def linear_grads(dL: np.ndarray, X: np.ndarray, W: np.ndarray):
    X64 = np.asarray(X, np.float64)
    W64 = np.asarray(W, np.float64)
    return dL @ W64, dL.T @ X64, dL.sum(axis=0)


def argmax_rows(z: np.ndarray) -> np.ndarray:
    """Lowest class index attaining the row maximum (numpy's argmax returns
    the first occurrence)."""
    if z.shape[1] == 0:
        return np.zeros(z.shape[0], dtype=np.int64)
    return z.argmax(axis=1).astype(np.int64)


def linear_cross_entropy(X, W, b, t, *, ignore_index: int = -100,
                         reduction: str = "mean", grad_scale: float = 1.0,
                         upstream=None, class_weight=None) -> dict:
    """The whole method on full arrays, unchunked.

    Returns loss (float for mean/sum, float64[N] for none), loss_rows,
    grad_X, grad_W, grad_b, lse, argmax, n_valid, n_bad, g and w (the
    per-row class weights).

    For reduction='none' with ``upstream`` given, the gradients are the
    backward of sum_n upstream[n] * loss_n ([LCE] reduction='none' backward,
    which recomputes the chunk loop with the upstream gradient folded into
    the row weights); with ``upstream`` None they are the gradients of
    sum_n loss_n.  ``class_weight`` ([V]) weighs each row by the weight of
    its target class, in the loss and in its denominator for mean."""
    X = np.asarray(X)
    W = np.asarray(W)
    V = W.shape[0]
    valid, bad, n_valid, n_bad = target_masks(t, V, ignore_index)
    tc = corrected_targets(t, valid)
    w = class_row_weights(valid, tc, class_weight)
    z = logits(X, W, b)
    lse = logsumexp_rows(z)
    loss_rows = row_losses(z, lse, tc, valid, w)
    loss = reduce_loss(loss_rows, w.sum(), reduction)
    g = row_weights(valid, reduction, grad_scale, upstream, tc=tc, class_weight=class_weight)
    dL = dlogits(z, lse, tc, g)
    gX, gW, gb = linear_grads(dL, X, W)
    return {"loss": loss, "loss_rows": loss_rows, "grad_X": gX,
            "grad_W": gW, "grad_b": gb, "lse": lse, "argmax": argmax_rows(z),
            "n_valid": n_valid, "n_bad": n_bad, "g": g, "w": w, "dL": dL}


def softmax_cross_entropy(z, t, *, ignore_index: int = -100,
                          reduction: str = "mean", grad_scale: float = 1.0,
                          class_weight=None):
    """Standalone CE on given logits ([LIG]): returns (loss, dL) where dL is
    what the in-place kernel writes over the logits buffer: the gradient of
    grad_scale * loss for mean / sum, of sum_n grad_scale * loss_n for none."""
    z = np.asarray(z, np.float64)
    V = z.shape[1]
    valid, _, _, _ = target_masks(t, V, ignore_index)
    tc = corrected_targets(t, valid)
    w = class_row_weights(valid, tc, class_weight)
    lse = logsumexp_rows(z)
    loss = reduce_loss(row_losses(z, lse, tc, valid, w), w.sum(), reduction)
    # 'none': the gradient of sum_n grad_scale * loss_n (the same upstream
    # value on every row).
    up = np.full(z.shape[0], grad_scale) if reduction == "none" else None
    g = row_weights(valid, reduction, grad_scale, up, tc=tc, class_weight=class_weight)
    return loss, dlogits(z, lse, tc, g)


# --------------------------------------------------------------------------
# Row-subset evaluation for shapes too large to hold the N x V logits.
# Every quantity above except the loss reductions and grad_W / grad_b is a
# function of one row; these helpers evaluate the same definitions on a
# subset of rows, and grad_W / grad_b columns as sums of per-row terms.
# --------------------------------------------------------------------------
def rows_forward(X_rows, W, b, t_rows, *, ignore_index: int = -100) -> dict:
    """lse, loss_n, argmax, the target logit and the row max for some rows."""
    V = np.asarray(W).shape[0]
    valid, _, _, _ = target_masks(t_rows, V, ignore_index)
    tc = corrected_targets(t_rows, valid)
    z = logits(X_rows, W, b)
    lse = logsumexp_rows(z)
    srt = np.sort(z, axis=1)
    gap = srt[:, -1] - srt[:, -2] if V > 1 else np.full(z.shape[0], np.inf)
    return {"lse": lse, "loss_rows": row_losses(z, lse, tc, valid),
            "argmax": argmax_rows(z), "top2_gap": gap, "rowmax": srt[:, -1]}


def rows_grad_x(X_rows, W, b, t_rows, g_rows, *, ignore_index: int = -100):
    """grad_X for some rows (each row of grad_X depends on that row only)."""
    V = np.asarray(W).shape[0]
    valid, _, _, _ = target_masks(t_rows, V, ignore_index)
    tc = corrected_targets(t_rows, valid)
    z = logits(X_rows, W, b)
    dL = dlogits(z, logsumexp_rows(z), tc, np.asarray(g_rows, np.float64))
    return dL @ np.asarray(W, np.float64)


def columns_grad_w_b(X_rows, W, b, t_rows, g_rows, cols, *,
                     ignore_index: int = -100):
    """The contribution of some rows to grad_W[cols] and grad_b[cols]:
    sum over those rows of dL[n, cols] X[n] and dL[n, cols]."""
    V = np.asarray(W).shape[0]
    valid, _, _, _ = target_masks(t_rows, V, ignore_index)
    tc = corrected_targets(t_rows, valid)
    z = logits(X_rows, W, b)
    dL = dlogits(z, logsumexp_rows(z), tc, np.asarray(g_rows, np.float64))
    dLc = dL[:, cols]
    return dLc.T @ np.asarray(X_rows, np.float64), dLc.sum(axis=0)


def row_block(X_rows, W, b, t_rows, g_rows, cols=None, *, ignore_index: int = -100,
              grad_x: bool = False, return_z: bool = False) -> dict:
    """All per-row quantities of a block of rows from one logits product:
    lse, loss_n, argmax, top-2 gap, row max; optionally the block's grad_X
    rows and its contribution to grad_W[cols] and grad_b[cols]; optionally
    the block's logits."""
    V = np.asarray(W).shape[0]
    valid, _, _, _ = target_masks(t_rows, V, ignore_index)
    tc = corrected_targets(t_rows, valid)
    z = logits(X_rows, W, b)
    lse = logsumexp_rows(z)
    out = {"lse": lse, "loss_rows": row_losses(z, lse, tc, valid), "argmax": argmax_rows(z)}
    part = np.partition(z, V - 2, axis=1)[:, V - 2:] if V > 1 else None
    out["rowmax"] = z.max(axis=1)
    out["top2_gap"] = (part[:, 1] - part[:, 0]) if V > 1 else np.full(z.shape[0], np.inf)
    if grad_x or cols is not None:
        dL = dlogits(z, lse, tc, np.asarray(g_rows, np.float64))
        if grad_x:
            out["grad_X"] = dL @ np.asarray(W, np.float64)
        if cols is not None:
            dLc = dL[:, cols]
            out["grad_W_cols"] = dLc.T @ np.asarray(X_rows, np.float64)
            out["grad_b_cols"] = dLc.sum(axis=0)
    if return_z:
        out["z"] = z
    return out
