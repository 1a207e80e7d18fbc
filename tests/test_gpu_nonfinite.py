"""NaN and -inf inputs behave as in the plain definition (IEEE arithmetic, no
masking beyond what the definition states).

- A NaN in one row n of X makes every logit of that row NaN: its loss is NaN
  (0 if the row is ignored, whose loss the definition sets to 0), its grad_X
  row is NaN, and every element of grad_W and grad_b is NaN, since the row's
  dL enters every sum over rows; for an ignored row that dL is 0 * NaN.
- A NaN in one row of W makes one logit of every row NaN, so every counted
  loss and every gradient element is NaN.
- The standalone CE: a NaN logit makes its row's loss and gradient row NaN.
- -inf logits (classes masked by a -inf bias) are softmax entries of exactly
  0: the losses stay finite and those classes' gradients are exactly 0.

The GPU's NaN positions must equal the oracle's, and its finite values meet
the usual tolerances.  The argmax of a row whose logits are all NaN is class
0 (numpy's first-NaN rule, the oracle's); with only some logits NaN it is
not specified, but it is a valid class."""
import numpy as np
import pytest

import lce_inputs as li
from gpu_common import (check_argmax, check_grad, check_loss, log, oracle, require_gpu,
                        run_ce, run_gpu)

pytestmark = pytest.mark.gpu

N, D, V = 600, 64, 1500


def _same_nans(got, ref, name):
    got, ref = np.asarray(got).reshape(-1), np.asarray(ref).reshape(-1)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref), err_msg=f"{name}: NaN positions")


def _finite_rows(ref_rows):
    return ~np.isnan(ref_rows).any(axis=tuple(range(1, ref_rows.ndim)))


def _check(gpu, ref, dt, reduction, z):
    assert int(gpu["n_valid"][0]) == ref["n_valid"]
    assert int(gpu["n_bad"][0]) == ref["n_bad"]
    _same_nans(gpu["loss"], ref["loss"], "loss")
    if reduction == "none":
        ok = ~np.isnan(ref["loss"])
        check_loss(gpu["loss"][ok], ref["loss"][ok], dt, "none")
    for key in ("grad_X", "grad_W", "grad_b"):
        _same_nans(gpu[key], ref[key], key)
        ok = _finite_rows(ref[key]) if ref[key].ndim > 1 else ~np.isnan(ref[key])
        if ok.any():
            check_grad(gpu[key][ok], ref[key][ok], dt, key)
    all_nan = np.isnan(z).all(axis=1)
    np.testing.assert_array_equal(gpu["argmax"][all_nan], 0)
    np.testing.assert_array_equal(ref["argmax"][all_nan], 0)
    assert np.all((gpu["argmax"] >= 0) & (gpu["argmax"] < z.shape[1]))
    rows = ~np.isnan(z).any(axis=1)
    zs = np.sort(z[rows], axis=1)
    check_argmax(gpu["argmax"][rows], ref["argmax"][rows], zs[:, -1] - zs[:, -2], zs[:, -1],
                 z[rows][np.arange(rows.sum()), gpu["argmax"][rows]])


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("chunk,group_rows", [(128, 0), (256, 512)])
def test_nan_in_one_row_of_x(dt, reduction, chunk, group_rows):
    """NaN in a counted row (in the second chunk) and in an ignored row (in
    the last, short chunk); 128-row chunks with the default groups, or
    256-row chunks two to a group (per-group statistics and combine)."""
    require_gpu()
    case = li.small_case(N, D, V, dtype=dt, seed=101, ignore_frac=0.0)
    X, t = case["X"].copy(), case["t"].copy()
    X[200, 5] = np.nan
    X[590, 17] = np.nan
    t[590] = li.IGNORE_INDEX
    t[[10, 400]] = li.IGNORE_INDEX
    up = case["u"] if reduction == "none" else None
    log(f"NaN in X rows dt={dt} {reduction} chunk={chunk} group_rows={group_rows}")
    gpu = run_gpu({**case, "X": X, "t": t}, dt, reduction=reduction, chunk_rows=chunk,
                  group_rows=group_rows, upstream=up)
    ref = oracle.linear_cross_entropy(X, case["W"], case["b"], t, reduction=reduction,
                                      upstream=up)
    assert np.isnan(ref["grad_W"]).all() and np.isnan(ref["grad_X"][[200, 590]]).all()
    _check(gpu, ref, dt, reduction, oracle.logits(X, case["W"], case["b"]))


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_nan_in_one_row_of_w(dt):
    require_gpu()
    case = li.small_case(N, D, V, dtype=dt, seed=102, ignore_frac=0.05)
    W = case["W"].copy()
    W[777, 3] = np.nan
    log(f"NaN in a W row dt={dt}")
    gpu = run_gpu({**case, "W": W}, dt, reduction="none", chunk_rows=128,
                  upstream=case["u"])
    ref = oracle.linear_cross_entropy(case["X"], W, case["b"], case["t"], reduction="none",
                                      upstream=case["u"])
    counted = case["t"] != li.IGNORE_INDEX
    assert np.isnan(ref["loss"][counted]).all() and np.isnan(ref["grad_X"]).all()
    _same_nans(gpu["loss"], ref["loss"], "loss")
    np.testing.assert_array_equal(gpu["loss"][~counted], 0.0)
    for key in ("grad_X", "grad_W", "grad_b"):
        _same_nans(gpu[key], ref[key], key)
    assert np.all((gpu["argmax"] >= 0) & (gpu["argmax"] < V))


def test_nan_logit_in_the_standalone_ce():
    require_gpu()
    rng = np.random.default_rng(103)
    n, v = 64, 4096
    z = rng.standard_normal((n, v)).astype(np.float32)
    z[9, 1234] = np.nan
    t = rng.integers(0, v, n).astype(np.int64)
    for reduction in ("mean", "none"):
        loss, nv, grad = run_ce(z, t, reduction=reduction)
        ref_loss, ref_grad = oracle.softmax_cross_entropy(z.astype(np.float64), t,
                                                          reduction=reduction)
        assert nv == n
        _same_nans(loss, ref_loss, "loss")
        _same_nans(grad, ref_grad, "gradient")
        ok = ~np.isnan(ref_grad).any(axis=1)
        check_grad(grad[ok], ref_grad[ok], "f32", "gradient")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("upstream", [True, False])
def test_a_whole_statistics_block_of_nan(dt, upstream):
    """W rows 128..255 NaN: the second 128-class statistics block of every
    row holds only NaN logits, whose NaN-skipping block max is -inf, like a
    block past V.  Its NaN sum must still reach every row (fp16 / fp32, and
    the bf16 loss-only forward, combine per-block maxima; the bf16 gradient
    path sums the blocks directly).  'none' with an upstream gradient
    (gradients) and without (the loss-only forward)."""
    require_gpu()
    case = li.small_case(N, D, V, dtype=dt, seed=104, ignore_frac=0.05)
    W = case["W"].copy()
    W[128:256] = np.nan
    up = case["u"] if upstream else None
    log(f"NaN statistics block dt={dt} upstream={upstream}")
    gpu = run_gpu({**case, "W": W}, dt, reduction="none", chunk_rows=128, upstream=up,
                  grads="xwb" if upstream else "")
    ref = oracle.linear_cross_entropy(case["X"], W, case["b"], case["t"], reduction="none",
                                      upstream=up)
    counted = case["t"] != li.IGNORE_INDEX
    assert np.isnan(ref["loss"][counted]).all()
    _same_nans(gpu["loss"], ref["loss"], "loss")
    np.testing.assert_array_equal(gpu["loss"][~counted], 0.0)
    assert np.all((gpu["argmax"] >= 0) & (gpu["argmax"] < V))
    if upstream:
        for key in ("grad_X", "grad_W", "grad_b"):
            _same_nans(gpu[key], ref[key], key)


@pytest.mark.parametrize("v", [4096, 8192, 65536, 160001])
def test_ce_row_nan_but_its_target(v):
    """A row NaN everywhere except the 4-class vector that holds its target.
    The two-pass kernel (V=160001) gives each thread a few dozen vectors, so
    all of the row's threads but one see NaN only and their NaN-skipping
    maxima stay -inf; the wave kernel (V=4096) and the on-chip ones (8192,
    65536) take one max over the row.  Either way the row's loss and
    gradient must be NaN and the other rows unchanged."""
    require_gpu()
    rng = np.random.default_rng(105)
    n = 32
    z = rng.standard_normal((n, v)).astype(np.float32)
    t = rng.integers(0, v, n).astype(np.int64)
    lo = 4 * (int(t[9]) // 4)
    keep = z[9, lo:lo + 4].copy()
    z[9] = np.nan
    z[9, lo:lo + 4] = keep
    loss, nv, grad = run_ce(z, t, reduction="none")
    ref_loss, ref_grad = oracle.softmax_cross_entropy(z.astype(np.float64), t, reduction="none")
    assert nv == n and np.isnan(ref_loss[9])
    _same_nans(loss, ref_loss, "loss")
    _same_nans(grad, ref_grad, "gradient")
    ok = ~np.isnan(ref_loss)
    check_loss(loss[ok], ref_loss[ok], "f32", "none")
    check_grad(grad[ok], ref_grad[ok], "f32", "gradient")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("reduction,grads", [("mean", "xwb"), ("none", "xwb"), ("none", "")])
def test_classes_masked_by_a_minus_inf_bias(dt, reduction, grads):
    """Classes masked with a -inf bias, no target among them: a whole
    128-class statistics block (256..383), a range inside another (700..719)
    and the last 30 classes of the ragged last tile.  Their logits are -inf,
    which the definition turns into softmax entries of exactly 0: every loss
    stays finite, the masked classes' grad_W rows and grad_b entries are
    exactly 0, and the rest meets the oracle's tolerances.  Gradients by
    mean and by 'none' with an upstream gradient, and the loss-only forward."""
    require_gpu()
    case = li.small_case(N, D, V, dtype=dt, seed=106, ignore_frac=0.05)
    masked = np.zeros(V, bool)
    masked[256:384] = masked[700:720] = masked[V - 30:] = True
    b = case["b"].copy()
    b[masked] = -np.inf
    t = case["t"].copy()
    t[(t >= 0) & masked[np.clip(t, 0, V - 1)]] = 1
    up = case["u"] if reduction == "none" and grads else None
    log(f"-inf bias dt={dt} {reduction} grads={grads!r}")
    gpu = run_gpu({**case, "b": b, "t": t}, dt, reduction=reduction, chunk_rows=128,
                  upstream=up, grads=grads)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], b, t, reduction=reduction,
                                      upstream=up)
    assert np.all(np.isfinite(ref["loss"])) and np.all(np.isfinite(gpu["loss"]))
    check_loss(gpu["loss"], ref["loss"], dt, reduction)
    if grads:
        for key in ("grad_X", "grad_W", "grad_b"):
            check_grad(gpu[key], ref[key], dt, key)
        assert np.all(gpu["grad_W"][masked] == 0.0) and np.all(gpu["grad_b"][masked] == 0.0)
    assert not np.any(masked[gpu["argmax"]])
