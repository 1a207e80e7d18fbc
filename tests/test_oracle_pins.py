"""Pins for the fp64 oracle: checks against what the mathematics fixes.

Each test pins the oracle to something other than itself: closed forms,
central finite differences, invariants the definition implies, and special
cases that reduce to an independent library routine (torch's CPU
cross_entropy in float64).  CPU only.
"""
import json
import math
import pathlib
import re

import numpy as np
import pytest
import torch

import oracle
from lce_inputs import small_case

RED = ["mean", "sum", "none"]
GOLDEN = pathlib.Path(__file__).parent / "golden"


def _case(N=6, D=4, V=9, seed=0, ignore_frac=0.2, bias=True, **kw):
    return small_case(N, D, V, seed=seed, ignore_frac=ignore_frac, bias=bias, **kw)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("V", [1000, 32000, 2, 7])
@pytest.mark.parametrize("reduction", RED)
def test_zero_weight_gives_log_v(V, reduction):
    """W = 0, b = 0: every logit is 0, so each counted row loses log V; the
    input gradient vanishes; grad_W and grad_b have closed forms; every row's
    argmax is class 0 (all classes tie, lowest index wins)."""
    N, D = 12, 5
    c = small_case(N, D, V, ignore_frac=0.25, bias=False, seed=3)
    W = np.zeros((V, D), np.float32)
    u = np.linspace(-1.0, 2.0, N)
    r = oracle.linear_cross_entropy(c["X"], W, np.zeros(V), c["t"],
                                    reduction=reduction, upstream=u)
    valid = c["t"] != -100
    nv = int(valid.sum())
    if reduction == "none":
        np.testing.assert_allclose(r["loss"], np.where(valid, math.log(V), 0.0),
                                   rtol=1e-15)
        g = np.where(valid, u, 0.0)
    else:
        expect = math.log(V) if reduction == "mean" else nv * math.log(V)
        assert abs(r["loss"] - expect) <= 1e-13 * expect
        g = np.where(valid, 1.0 / nv if reduction == "mean" else 1.0, 0.0)
    assert np.all(r["grad_X"] == 0.0)
    X = c["X"].astype(np.float64)
    tc = np.where(valid, c["t"], 0)
    gW = np.zeros((V, D))
    gb = np.zeros(V)
    for n in range(N):
        gW += g[n] * X[n][None, :] / V
        gb += g[n] / V
        gW[tc[n]] -= g[n] * X[n]
        gb[tc[n]] -= g[n]
    np.testing.assert_allclose(r["grad_W"], gW, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["grad_b"], gb, rtol=1e-12, atol=1e-15)
    assert np.all(r["argmax"] == 0)


def test_two_classes_is_softplus():
    """V = 2: loss_n = log(1 + exp(z_other - z_target))."""
    c = _case(N=40, D=3, V=2, ignore_frac=0.0, seed=5)
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="none")
    X, W, b = (c[k].astype(np.float64) for k in ("X", "W", "b"))
    for n in range(40):
        z = [sum(X[n, k] * W[j, k] for k in range(3)) + b[j] for j in range(2)]
        tn = c["t"][n]
        expect = math.log1p(math.exp(z[1 - tn] - z[tn]))
        assert abs(r["loss"][n] - expect) <= 1e-14 * max(1.0, expect)


def _closed_form(expr):
    """Evaluate a fixture's closed-form expression in e (nothing else allowed)."""
    assert re.fullmatch(r"[0-9e()+\-*/ .log]+", expr), expr
    return eval(expr, {"__builtins__": {}}, {"log": math.log, "e": math.e})


def test_hand_worked_example():
    """The 2x2x3 case worked by hand in tests/golden (its derivation and
    sources are in the fixture)."""
    fx = json.loads((GOLDEN / "hand_worked_example.json").read_text())
    inp, exp = fx["inputs"], fx["expect"]
    r = oracle.linear_cross_entropy(np.array(inp["X"], float), np.array(inp["W"], float),
                                    np.array(inp["b"], float), np.array(inp["t"]),
                                    reduction=inp["reduction"])
    ev = np.vectorize(_closed_form, otypes=[float])
    assert abs(r["loss"] - _closed_form(exp["loss"])) < 1e-15
    np.testing.assert_allclose(r["loss_rows"], ev(exp["loss_rows"]), rtol=1e-15)
    for k in ("grad_b", "grad_X", "grad_W"):
        np.testing.assert_allclose(r[k], ev(np.array(exp[k])), rtol=1e-14, atol=1e-16)
    assert list(r["argmax"]) == exp["argmax"]


# -------------------------------------------------- an independent library
@pytest.mark.parametrize("reduction", RED)
@pytest.mark.parametrize("ignore_index", [-100, 3])
def test_matches_torch_cpu_cross_entropy(reduction, ignore_index):
    """Special case that reduces to a library routine: torch's float64 CPU
    cross_entropy on X W^T + b, with autograd for the three gradients."""
    c = small_case(23, 6, 11, seed=11, ignore_frac=0.2, ignore_index=ignore_index)
    X = torch.tensor(c["X"], dtype=torch.float64, requires_grad=True)
    W = torch.tensor(c["W"], dtype=torch.float64, requires_grad=True)
    b = torch.tensor(c["b"], dtype=torch.float64, requires_grad=True)
    t = torch.tensor(c["t"])
    loss = torch.nn.functional.cross_entropy(X @ W.T + b, t, ignore_index=ignore_index,
                                             reduction=reduction)
    u = torch.tensor(c["u"], dtype=torch.float64)
    (loss * u).sum().backward() if reduction == "none" else loss.backward()
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"],
                                    ignore_index=ignore_index, reduction=reduction,
                                    upstream=c["u"])
    np.testing.assert_allclose(r["loss"], loss.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(r["grad_X"], X.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"], W.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["grad_b"], b.grad.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 1.5])
def test_standalone_ce_matches_torch(scale):
    rng = np.random.default_rng(7)
    z = rng.standard_normal((17, 13))
    t = rng.integers(0, 13, 17)
    t[[2, 9]] = -100
    zt = torch.tensor(z, requires_grad=True)
    for red in RED:
        zt.grad = None
        loss = torch.nn.functional.cross_entropy(zt, torch.tensor(t), reduction=red)
        (scale * (loss.sum() if red == "none" else loss)).backward()
        ol, dL = oracle.softmax_cross_entropy(z, t, reduction=red, grad_scale=scale)
        np.testing.assert_allclose(ol, loss.detach().numpy(), rtol=1e-13)
        np.testing.assert_allclose(dL, zt.grad.numpy(), rtol=1e-12, atol=1e-16)


# ------------------------------------------------------- finite differences
def _scalar_objective(X, W, b, t, reduction, u):
    r = oracle.linear_cross_entropy(X, W, b, t, reduction=reduction)
    if reduction == "none":
        return float(np.dot(u, r["loss"]))
    return r["loss"]


@pytest.mark.parametrize("reduction", RED)
def test_central_finite_differences(reduction):
    """Tiny shape (N=5, D=3, V=7, one ignored row): every gradient entry
    agrees with a central difference of the loss."""
    c = small_case(5, 3, 7, seed=2, ignore_frac=0.2, x_std=0.7, w_std=0.9)
    X, W, b = (c[k].astype(np.float64) for k in ("X", "W", "b"))
    t, u = c["t"], c["u"].astype(np.float64)
    assert (t == -100).sum() == 1
    r = oracle.linear_cross_entropy(X, W, b, t, reduction=reduction, upstream=u)
    for name, arr, grad in (("X", X, r["grad_X"]), ("W", W, r["grad_W"]),
                            ("b", b, r["grad_b"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            args = {"X": X, "W": W, "b": b}
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            fp = _scalar_objective(**{**args, name: p}, t=t, reduction=reduction, u=u)
            fm = _scalar_objective(**{**args, name: m}, t=t, reduction=reduction, u=u)
            fd[idx] = (fp - fm) / (2 * h)
        scale = max(1e-3, np.abs(grad).max())
        assert np.abs(fd - grad).max() <= 1e-7 * scale, name


# --------------------------------------------------------------- invariants
def test_dlogit_rows_sum_to_zero():
    c = _case(N=30, D=8, V=50, seed=4)
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum")
    np.testing.assert_allclose(r["dL"].sum(axis=1), 0.0, atol=1e-15)
    np.testing.assert_allclose(r["grad_b"].sum(), 0.0, atol=1e-13)
    np.testing.assert_allclose(r["grad_W"].sum(axis=0), 0.0, atol=1e-13)


def test_ignored_rows_contribute_nothing():
    c = _case(N=20, D=6, V=30, seed=6, ignore_frac=0.3)
    ign = c["t"] == -100
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    assert np.all(r["loss_rows"][ign] == 0.0)
    assert np.all(r["grad_X"][ign] == 0.0)
    X2 = c["X"].copy()
    X2[ign] = 123.0        # changing an ignored row changes nothing else
    r2 = oracle.linear_cross_entropy(X2, c["W"], c["b"], c["t"], reduction="mean")
    assert r2["loss"] == r["loss"]
    np.testing.assert_array_equal(r2["grad_X"][~ign], r["grad_X"][~ign])
    np.testing.assert_allclose(r2["grad_W"], r["grad_W"], rtol=1e-13, atol=1e-16)
    np.testing.assert_array_equal(r2["grad_b"], r["grad_b"])


def test_mean_is_sum_over_count():
    c = _case(N=25, D=5, V=17, seed=8, ignore_frac=0.2)
    rm = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    rs = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum")
    nv = int((c["t"] != -100).sum())
    assert rm["n_valid"] == nv == 20
    assert abs(rm["loss"] - rs["loss"] / nv) <= 1e-15 * abs(rm["loss"])
    for k in ("grad_X", "grad_W", "grad_b"):
        np.testing.assert_allclose(rm[k], rs[k] / nv, rtol=1e-13, atol=1e-17)


def test_all_ignored_and_empty():
    c = _case(N=8, D=4, V=10, seed=9, ignore_frac=1.0)
    rm = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    assert math.isnan(rm["loss"])
    for k in ("grad_X", "grad_W", "grad_b"):
        assert np.all(np.isnan(rm[k]))
    rs = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum")
    assert rs["loss"] == 0.0
    for k in ("grad_X", "grad_W", "grad_b"):
        assert np.all(rs[k] == 0.0)
    X0 = np.zeros((0, 4))
    t0 = np.zeros(0, np.int64)
    e = oracle.linear_cross_entropy(X0, c["W"], c["b"], t0, reduction="mean")
    assert math.isnan(e["loss"]) and e["grad_X"].shape == (0, 4)
    assert np.all(e["grad_W"] == 0) and np.all(e["grad_b"] == 0)
    e = oracle.linear_cross_entropy(X0, c["W"], c["b"], t0, reduction="sum")
    assert e["loss"] == 0.0


def test_bias_shift_invariance():
    c = _case(N=15, D=4, V=12, seed=10)
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    r2 = oracle.linear_cross_entropy(c["X"], c["W"], c["b"].astype(np.float64) + 3.25,
                                     c["t"], reduction="mean")
    assert abs(r["loss"] - r2["loss"]) < 1e-13
    for k in ("grad_X", "grad_W", "grad_b"):
        np.testing.assert_allclose(r[k], r2[k], rtol=1e-11, atol=1e-14)


def test_large_logits_stay_finite():
    """Logits near 1e4: the max-shift keeps everything finite and the loss
    is close to max logit - target logit."""
    c = _case(N=10, D=4, V=8, seed=12, ignore_frac=0.0)
    X = c["X"].astype(np.float64) * 1e4
    r = oracle.linear_cross_entropy(X, c["W"], c["b"], c["t"], reduction="none")
    assert np.all(np.isfinite(r["loss"])) and np.all(np.isfinite(r["grad_W"]))
    z = oracle.logits(X, c["W"], c["b"])
    approx = z.max(1) - z[np.arange(10), c["t"]]
    assert np.all(r["loss"] >= approx - 1e-9)
    assert np.all(r["loss"] <= approx + math.log(8) + 1e-9)


def test_none_backward_with_unit_upstream_equals_sum():
    c = _case(N=14, D=5, V=9, seed=13)
    rn = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="none",
                                     upstream=np.ones(14))
    rs = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum")
    for k in ("grad_X", "grad_W", "grad_b"):
        np.testing.assert_allclose(rn[k], rs[k], rtol=1e-14, atol=1e-17)
    assert abs(rn["loss"].sum() - rs["loss"]) < 1e-12


def test_grad_scale_is_linear():
    c = _case(N=11, D=3, V=6, seed=14)
    r1 = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    r2 = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean",
                                     grad_scale=-2.5)
    assert r1["loss"] == r2["loss"]
    for k in ("grad_X", "grad_W", "grad_b"):
        np.testing.assert_allclose(r2[k], -2.5 * r1[k], rtol=1e-14, atol=1e-17)


def test_bad_targets_are_counted_and_ignored():
    c = _case(N=10, D=3, V=5, seed=15, ignore_frac=0.1)
    t = c["t"].copy()
    t[[1, 4]] = [5, -7]               # out of range and not ignore_index
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], t, reduction="mean")
    assert r["n_bad"] == 2 and r["n_valid"] == 10 - 1 - 2
    assert np.all(r["grad_X"][[1, 4]] == 0.0) and np.all(r["loss_rows"][[1, 4]] == 0.0)


def test_ignore_index_inside_range():
    c = _case(N=30, D=4, V=6, seed=16, ignore_frac=0.0)
    t = c["t"]
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], t, ignore_index=2,
                                    reduction="sum")
    assert r["n_valid"] == int((t != 2).sum())
    assert np.all(r["loss_rows"][t == 2] == 0) and np.all(r["grad_X"][t == 2] == 0)


def test_argmax_brute_force_and_ties():
    c = _case(N=9, D=3, V=6, seed=17)
    W = c["W"].astype(np.float64)
    W[4] = W[1]                      # classes 1 and 4 always tie
    r = oracle.linear_cross_entropy(c["X"], W, None, c["t"], reduction="sum")
    X = c["X"].astype(np.float64)
    for n in range(9):
        zs = [sum(X[n, k] * W[j, k] for k in range(3)) for j in range(6)]
        best = 0
        for j in range(1, 6):
            if zs[j] > zs[best]:
                best = j
        assert r["argmax"][n] == best
        assert r["argmax"][n] != 4


# ------------------------------------------- row-subset helpers vs the whole
def test_row_subset_helpers_agree_with_full():
    c = _case(N=40, D=6, V=25, seed=18)
    full = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean")
    rows = np.array([0, 7, 13, 39])
    f = oracle.rows_forward(c["X"][rows], c["W"], c["b"], c["t"][rows])
    np.testing.assert_allclose(f["lse"], full["lse"][rows], rtol=1e-15)
    np.testing.assert_allclose(f["loss_rows"], full["loss_rows"][rows], rtol=1e-15)
    np.testing.assert_array_equal(f["argmax"], full["argmax"][rows])
    gx = oracle.rows_grad_x(c["X"][rows], c["W"], c["b"], c["t"][rows], full["g"][rows])
    np.testing.assert_allclose(gx, full["grad_X"][rows], rtol=1e-13, atol=1e-17)
    cols = np.array([1, 5, 24])
    gw = np.zeros((3, 6))
    gb = np.zeros(3)
    for r0 in range(0, 40, 16):
        sl = slice(r0, r0 + 16)
        a, bb = oracle.columns_grad_w_b(c["X"][sl], c["W"], c["b"], c["t"][sl],
                                        full["g"][sl], cols)
        gw += a
        gb += bb
    np.testing.assert_allclose(gw, full["grad_W"][cols], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(gb, full["grad_b"][cols], rtol=1e-12, atol=1e-16)


def test_row_block_agrees_with_full():
    c = _case(N=40, D=6, V=25, seed=19)
    full = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum")
    cols = np.array([0, 3, 24])
    gw = np.zeros((3, 6))
    gb = np.zeros(3)
    for r0 in range(0, 40, 11):
        sl = slice(r0, r0 + 11)
        r = oracle.row_block(c["X"][sl], c["W"], c["b"], c["t"][sl], full["g"][sl], cols,
                             grad_x=True, return_z=True)
        np.testing.assert_allclose(r["lse"], full["lse"][sl], rtol=1e-15)
        np.testing.assert_allclose(r["loss_rows"], full["loss_rows"][sl], rtol=1e-15)
        np.testing.assert_allclose(r["grad_X"], full["grad_X"][sl], rtol=1e-13, atol=1e-17)
        np.testing.assert_array_equal(r["argmax"], full["argmax"][sl])
        zs = np.sort(r["z"], axis=1)
        np.testing.assert_allclose(r["top2_gap"], zs[:, -1] - zs[:, -2], rtol=1e-15)
        gw += r["grad_W_cols"]
        gb += r["grad_b_cols"]
    np.testing.assert_allclose(gw, full["grad_W"][cols], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(gb, full["grad_b"][cols], rtol=1e-12, atol=1e-16)


# ------------------------------------------------------- per-class weights
# [LCE] _ChunkContext.neg_weight_target: a row weighs weight[target]; mean
# divides by the sum of the unmasked row weights (NaN when it is 0).
def _cw(V, seed=31):
    return np.random.default_rng(seed).uniform(0.2, 3.0, V)


@pytest.mark.parametrize("reduction", RED)
@pytest.mark.parametrize("ignore_index", [-100, 3])
def test_class_weights_match_torch(reduction, ignore_index):
    c = small_case(23, 6, 11, seed=32, ignore_frac=0.2, ignore_index=ignore_index)
    cw = _cw(11)
    X = torch.tensor(c["X"], dtype=torch.float64, requires_grad=True)
    W = torch.tensor(c["W"], dtype=torch.float64, requires_grad=True)
    b = torch.tensor(c["b"], dtype=torch.float64, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(X @ W.T + b, torch.tensor(c["t"]), weight=torch.tensor(cw),
                                             ignore_index=ignore_index, reduction=reduction)
    u = torch.tensor(c["u"], dtype=torch.float64)
    (loss * u).sum().backward() if reduction == "none" else loss.backward()
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], ignore_index=ignore_index,
                                    reduction=reduction, upstream=c["u"], class_weight=cw)
    np.testing.assert_allclose(r["loss"], loss.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(r["grad_X"], X.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"], W.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["grad_b"], b.grad.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("reduction", RED)
def test_unit_class_weights_change_nothing(reduction):
    c = _case(N=12, D=5, V=8, seed=33)
    a = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction=reduction)
    w = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction=reduction,
                                    class_weight=np.ones(8))
    for k in ("loss", "grad_X", "grad_W", "grad_b"):
        np.testing.assert_array_equal(a[k], w[k])


def test_mean_is_invariant_to_scaling_the_class_weights():
    c = _case(N=14, D=5, V=9, seed=34)
    cw = _cw(9)
    a = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], class_weight=cw)
    s = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], class_weight=cw * 7.5)
    assert abs(a["loss"] - s["loss"]) <= 1e-14 * abs(a["loss"])
    for k in ("grad_X", "grad_W", "grad_b"):
        np.testing.assert_allclose(a[k], s[k], rtol=1e-13, atol=1e-16)


def test_weighted_sum_is_the_weighted_row_losses():
    """sum with class weights = sum_n w[t_n] loss_n of the unweighted rows,
    and mean divides that by sum_n w[t_n] over counted rows."""
    c = _case(N=15, D=4, V=7, seed=35)
    cw = _cw(7)
    rows = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="none")
    valid, _, _, _ = oracle.target_masks(c["t"], 7, -100)
    wrow = np.where(valid, cw[np.where(valid, c["t"], 0)], 0.0)
    s = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum", class_weight=cw)
    m = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="mean", class_weight=cw)
    assert abs(s["loss"] - float(np.dot(wrow, rows["loss"]))) < 1e-12
    assert abs(m["loss"] - s["loss"] / wrow.sum()) < 1e-13


def test_zero_total_class_weight():
    """mean: every counted row weighs 0 -> NaN loss and gradients (the pages
    divide by NaN when the weight sum is 0); sum: loss 0, gradients 0."""
    c = _case(N=10, D=4, V=6, seed=36)
    cw = np.zeros(6)
    m = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], class_weight=cw)
    assert math.isnan(m["loss"]) and np.all(np.isnan(m["grad_X"]))
    s = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], reduction="sum", class_weight=cw)
    assert s["loss"] == 0.0 and np.all(s["grad_X"] == 0.0) and np.all(s["grad_W"] == 0.0)


def test_weighted_mean_finite_differences():
    c = _case(N=5, D=3, V=7, seed=37)
    cw = _cw(7)
    r = oracle.linear_cross_entropy(c["X"], c["W"], c["b"], c["t"], class_weight=cw)
    X = c["X"].astype(np.float64)
    for (i, j) in [(0, 0), (2, 1), (4, 2)]:
        h = 1e-6 * max(1.0, abs(X[i, j]))
        Xp, Xm = X.copy(), X.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        lp = oracle.linear_cross_entropy(Xp, c["W"], c["b"], c["t"], class_weight=cw)["loss"]
        lm = oracle.linear_cross_entropy(Xm, c["W"], c["b"], c["t"], class_weight=cw)["loss"]
        assert abs((lp - lm) / (2 * h) - r["grad_X"][i, j]) <= 1e-7 * max(1.0, abs(r["grad_X"][i, j]))


@pytest.mark.parametrize("reduction", RED)
def test_standalone_ce_class_weights_match_torch(reduction):
    rng = np.random.default_rng(38)
    z = rng.standard_normal((17, 13))
    t = rng.integers(0, 13, 17)
    t[[2, 9]] = -100
    cw = _cw(13, 39)
    zt = torch.tensor(z, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(zt, torch.tensor(t), weight=torch.tensor(cw),
                                             reduction=reduction)
    (loss.sum() * 1.5).backward()
    l, dl = oracle.softmax_cross_entropy(z, t, reduction=reduction, grad_scale=1.5, class_weight=cw)
    np.testing.assert_allclose(l, loss.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(dl, zt.grad.numpy(), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ NaN propagation
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_nan_rows_propagate_as_in_torch(reduction):
    """A NaN in one counted input row and in one ignored row: the oracle's
    loss and gradients hold NaN exactly where torch's float64 cross_entropy
    with autograd does (the ignored row's loss stays 0, its dL is 0 * NaN),
    and equal torch's values elsewhere."""
    case = _case(N=8, D=5, V=11, seed=4, ignore_frac=0.0)
    X, t = case["X"].astype(np.float64), case["t"].copy()
    X[2, 1] = np.nan
    X[5, 3] = np.nan
    t[5] = -100
    ref = oracle.linear_cross_entropy(X, case["W"], case["b"], t, reduction=reduction,
                                      upstream=np.ones(8) if reduction == "none" else None)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(case["W"], dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(case["b"], dtype=torch.float64, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Xt @ Wt.T + bt, torch.tensor(t),
                                             ignore_index=-100, reduction=reduction)
    (loss.sum() if reduction == "none" else loss).backward()
    got = {"loss": loss.detach().numpy(), "grad_X": Xt.grad.numpy(),
           "grad_W": Wt.grad.numpy(), "grad_b": bt.grad.numpy()}
    for k, v in got.items():
        r = np.asarray(ref[k], np.float64).reshape(np.shape(v))
        np.testing.assert_array_equal(np.isnan(r), np.isnan(v), err_msg=k)
        ok = ~np.isnan(v)
        np.testing.assert_allclose(r[ok], v[ok], rtol=1e-12, atol=1e-12, err_msg=k)
    assert np.isnan(got["grad_W"]).all() and np.isnan(got["grad_X"][[2, 5]]).all()
    if reduction == "none":
        assert np.isnan(got["loss"][2]) and got["loss"][5] == 0.0


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_standalone_ce_nan_row_as_in_torch(reduction):
    """A NaN logit in one row: the standalone CE's loss and in-place gradient
    hold NaN where torch's float64 cross_entropy with autograd does."""
    rng = np.random.default_rng(12)
    z = rng.standard_normal((6, 13))
    z[3, 7] = np.nan
    t = rng.integers(0, 13, 6)
    loss, dl = oracle.softmax_cross_entropy(z, t, reduction=reduction)
    zt = torch.tensor(z, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(t), reduction=reduction)
    (lt.sum() if reduction == "none" else lt).backward()
    for got, want, name in ((np.atleast_1d(loss), np.atleast_1d(lt.detach().numpy()), "loss"),
                            (dl, zt.grad.numpy(), "gradient")):
        np.testing.assert_array_equal(np.isnan(got), np.isnan(want), err_msg=name)
        ok = ~np.isnan(want)
        np.testing.assert_allclose(got[ok], want[ok], rtol=1e-12, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_standalone_ce_masked_logits_as_in_torch(reduction):
    """Logits masked to -inf (a class range of every row, and all but two
    classes of one row; no target among them): the loss stays finite and
    the masked classes' gradient is exactly 0, as in torch's float64
    cross_entropy with autograd."""
    rng = np.random.default_rng(13)
    z = rng.standard_normal((6, 16))
    z[:, 4:12] = -np.inf
    z[2, 13:] = -np.inf
    t = np.array([0, 1, 12, 13, 14, 15])
    loss, dl = oracle.softmax_cross_entropy(z, t, reduction=reduction)
    zt = torch.tensor(z, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(t), reduction=reduction)
    (lt.sum() if reduction == "none" else lt).backward()
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(dl))
    assert np.all(dl[:, 4:12] == 0.0) and np.all(dl[2, 13:] == 0.0)
    np.testing.assert_allclose(np.atleast_1d(loss), np.atleast_1d(lt.detach().numpy()),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dl, zt.grad.numpy(), rtol=1e-12, atol=1e-12)
