"""Planted mistakes: each mutant below is a plausible slip in the oracle
(a dropped term, a wrong sign, index or operand, a wrong denominator).  The
pins must reject every one of them.  The mistakes are planted in the oracle,
on the CPU, through monkeypatching; nothing here touches the GPU path."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.lce_oracle as lo
from lce_inputs import small_case


def _pin_torch(reduction="mean", ignore_index=-100):
    c = small_case(13, 5, 9, seed=21, ignore_frac=0.25, ignore_index=ignore_index)
    X = torch.tensor(c["X"], dtype=torch.float64, requires_grad=True)
    W = torch.tensor(c["W"], dtype=torch.float64, requires_grad=True)
    b = torch.tensor(c["b"], dtype=torch.float64, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(X @ W.T + b, torch.tensor(c["t"]),
                                             ignore_index=ignore_index,
                                             reduction=reduction)
    u = torch.tensor(c["u"], dtype=torch.float64)
    (loss * u).sum().backward() if reduction == "none" else loss.backward()
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction=reduction,
                                    ignore_index=ignore_index, upstream=c["u"])
    return (np.allclose(r["loss"], loss.detach().numpy(), rtol=1e-12)
            and np.allclose(r["grad_X"], X.grad.numpy(), rtol=1e-10, atol=1e-14)
            and np.allclose(r["grad_W"], W.grad.numpy(), rtol=1e-10, atol=1e-14)
            and np.allclose(r["grad_b"], b.grad.numpy(), rtol=1e-10, atol=1e-14))


def _pin_torch_class_weight(reduction="mean"):
    """Per-class weights against torch's cross_entropy(weight=...)."""
    c = small_case(13, 5, 9, seed=26, ignore_frac=0.25)
    cw = np.random.default_rng(27).uniform(0.2, 3.0, 9)
    X = torch.tensor(c["X"], dtype=torch.float64, requires_grad=True)
    W = torch.tensor(c["W"], dtype=torch.float64, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(X @ W.T, torch.tensor(c["t"]),
                                             weight=torch.tensor(cw), reduction=reduction)
    u = torch.tensor(c["u"], dtype=torch.float64)
    (loss * u).sum().backward() if reduction == "none" else loss.backward()
    r = oracle.linear_cross_entropy(c["X"], c["W"], None, c["t"], reduction=reduction,
                                    upstream=c["u"], class_weight=cw)
    return (np.allclose(r["loss"], loss.detach().numpy(), rtol=1e-12)
            and np.allclose(r["grad_X"], X.grad.numpy(), rtol=1e-10, atol=1e-14)
            and np.allclose(r["grad_W"], W.grad.numpy(), rtol=1e-10, atol=1e-14))


def _pin_zero_weight():
    c = small_case(10, 4, 7, seed=22, ignore_frac=0.2, bias=False)
    r = oracle.linear_cross_entropy(c["X"], np.zeros((7, 4)), None, c["t"])
    return abs(r["loss"] - math.log(7)) < 1e-13 and np.all(r["argmax"] == 0)


def _pin_all_ignored():
    c = small_case(6, 3, 5, seed=23, ignore_frac=1.0)
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    return math.isnan(r["loss"]) and np.all(np.isnan(r["grad_W"]))


def _pin_argmax():
    c = small_case(8, 3, 6, seed=24)
    W = c["W"].astype(np.float64)
    W[4] = W[1]
    r = oracle.linear_cross_entropy(c["X"], W, None, c["t"], reduction="sum")
    z = c["X"].astype(np.float64) @ W.T
    return all(r["argmax"][n] == min(j for j in range(6) if z[n, j] == z[n].max())
               for n in range(8))


def _pin_bad_targets():
    c = small_case(8, 3, 5, seed=25, ignore_frac=0.0)
    t = c["t"].copy()
    t[2] = 9
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], t, reduction="mean")
    return r["n_bad"] == 1 and r["n_valid"] == 7 and np.all(r["grad_X"][2] == 0)


def _all_pins():
    return (all(_pin_torch(red, ii) for red in ("mean", "sum", "none")
                for ii in (-100, 2))
            and all(_pin_torch_class_weight(red) for red in ("mean", "sum", "none"))
            and _pin_zero_weight() and _pin_all_ignored() and _pin_argmax()
            and _pin_bad_targets())


def test_unmutated_oracle_passes_every_pin():
    assert _all_pins()


def _m_dlogits_no_onehot(z, lse, tc, g):
    return g[:, None] * np.exp(z - lse[:, None])


def _m_dlogits_sign(z, lse, tc, g):
    return -_ORIG["dlogits"](z, lse, tc, g)


def _m_grads_transposed(dL, X, W):
    """grad_W pairs dL rows with the wrong X rows (reversed row order)."""
    gx, _, gb = _ORIG["linear_grads"](dL, X, W)
    return gx, dL[::-1].T @ np.asarray(X, np.float64), gb


def _m_grad_x_uses_x(dL, X, W):
    """grad_X formed from the wrong operand's columns (W's rows reversed)."""
    _, gw, gb = _ORIG["linear_grads"](dL, X, W)
    return dL @ np.asarray(W, np.float64)[::-1], gw, gb


def _m_lse_no_log(z):
    m = z.max(axis=1)
    return m + np.exp(z - m[:, None]).sum(axis=1)


def _m_lse_no_shift_back(z):
    m = z.max(axis=1)
    return np.log(np.exp(z - m[:, None]).sum(axis=1))


def _m_mean_over_N(valid, reduction, grad_scale=1.0, upstream=None, **kw):
    if reduction == "mean":
        w = lo.class_row_weights(valid, kw.get("tc"), kw.get("class_weight"))
        return w * grad_scale / len(valid)
    return _ORIG["row_weights"](valid, reduction, grad_scale, upstream, **kw)


def _m_ignore_weights(valid, reduction, grad_scale=1.0, upstream=None, **kw):
    return _ORIG["row_weights"](np.ones_like(valid), reduction, grad_scale, upstream, **kw)


def _m_mean_over_count(valid, reduction, grad_scale=1.0, upstream=None, **kw):
    """Class weights in the numerator, the row count as the denominator."""
    if reduction == "mean":
        w = lo.class_row_weights(valid, kw.get("tc"), kw.get("class_weight"))
        return w * grad_scale / valid.sum()
    return _ORIG["row_weights"](valid, reduction, grad_scale, upstream, **kw)


def _m_class_weight_dropped(valid, reduction, grad_scale=1.0, upstream=None, **kw):
    kw = dict(kw, class_weight=None)
    return _ORIG["row_weights"](valid, reduction, grad_scale, upstream, **kw)


def _m_mask_after_correction(t, V, ignore_index):
    t = np.asarray(t, np.int64)
    tc = np.where((t < 0) | (t >= V), 0, t)
    ignored = tc == ignore_index
    valid = ~ignored
    return valid, np.zeros_like(valid), int(valid.sum()), 0


def _m_bias_dropped(X, W, b):
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64).T


def _m_argmax_last(z):
    return (z.shape[1] - 1 - z[:, ::-1].argmax(axis=1)).astype(np.int64)


def _m_loss_target_index_off_by_one(z, lse, tc, valid, w=None):
    n = np.arange(z.shape[0])
    loss = np.where(valid, lse - z[n, np.minimum(tc + 1, z.shape[1] - 1)], 0.0)
    return loss if w is None else w * loss


def _m_loss_unweighted(z, lse, tc, valid, w=None):
    return _ORIG["row_losses"](z, lse, tc, valid)


_ORIG = {k: getattr(lo, k) for k in ("dlogits", "linear_grads", "logsumexp_rows",
                                      "row_weights", "target_masks", "logits",
                                      "argmax_rows", "row_losses")}

MUTANTS = [
    ("dlogits", _m_dlogits_no_onehot),
    ("dlogits", _m_dlogits_sign),
    ("linear_grads", _m_grads_transposed),
    ("linear_grads", _m_grad_x_uses_x),
    ("logsumexp_rows", _m_lse_no_log),
    ("logsumexp_rows", _m_lse_no_shift_back),
    ("row_weights", _m_mean_over_N),
    ("row_weights", _m_ignore_weights),
    ("target_masks", _m_mask_after_correction),
    ("logits", _m_bias_dropped),
    ("argmax_rows", _m_argmax_last),
    ("row_losses", _m_loss_target_index_off_by_one),
    ("row_weights", _m_mean_over_count),
    ("row_weights", _m_class_weight_dropped),
    ("row_losses", _m_loss_unweighted),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_reject_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(lo, name, mutant)
    with np.errstate(all="ignore"):
        try:
            ok = _all_pins()
        except (FloatingPointError, ValueError, IndexError, ZeroDivisionError):
            ok = False       # a numerical failure in the mutant is a rejection too
    assert not ok, f"pins did not catch mutant {mutant.__name__}"
