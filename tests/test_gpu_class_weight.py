"""GPU parity of per-class cross-entropy weights against the fp64 oracle: the
fused path (fp32, bf16 and fp16, every reduction, ignored and out-of-range rows,
classes of weight 0, ragged chunks) and the standalone in-place CE (streamed
and on-chip rows).  With weights the mean divides by the sum of the counted
rows' weights; a zero weight sum makes the mean loss and every gradient NaN.
Unit weights must reproduce the unweighted run bit for bit."""
import math

import numpy as np
import pytest

import lce_inputs as li
from gpu_common import check_all, log, oracle, rel_err, require_gpu, run_ce, run_gpu

pytestmark = pytest.mark.gpu


def _ref(case, cw, reduction="mean", upstream=None, grad_scale=1.0, ignore_index=-100):
    return oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                       ignore_index=ignore_index, reduction=reduction,
                                       upstream=upstream, grad_scale=grad_scale,
                                       class_weight=cw)


def _z(case):
    return oracle.logits(case["X"], case["W"], case["b"])


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_fused_class_weights(dt, reduction):
    """N=333 rows in chunks of 70 (a ragged last chunk), V=777 (a ragged last
    tile), 15% ignored rows, a tenth of the classes weighted 0."""
    require_gpu()
    case = li.small_case(333, 128, 777, dtype=dt, seed=21, ignore_frac=0.15)
    cw = li.class_weights(777, seed=21, zero_frac=0.1)
    up = case["u"] if reduction == "none" else None
    log(f"class weights dt={dt} reduction={reduction}")
    gpu = run_gpu(case, dt, reduction=reduction, chunk_rows=70, upstream=up, grad_scale=0.75,
                  class_weight=cw)
    ref = _ref(case, cw, reduction, upstream=up, grad_scale=0.75)
    errs = check_all(gpu, ref, dt, reduction, z=_z(case))
    zero_rows = (case["t"] >= 0) & (cw[np.clip(case["t"], 0, None)] == 0.0)
    assert zero_rows.any()
    assert np.all(gpu["grad_X"][zero_rows] == 0.0)
    if reduction == "none":
        assert np.all(gpu["loss"][zero_rows] == 0.0)
    log(f"class weights errors {errs}")


def test_mid_bf16_class_weights():
    """The mid bf16 workload (N=4096, D=2048, V=32000, 1024-row chunks) with
    per-class weights: many logits tiles, the weighted mean."""
    require_gpu()
    cfg = li.MID_BF16
    case = li.lce_inputs(cfg)
    cw = li.class_weights(cfg.V, seed=cfg.seed, zero_frac=0.05)
    log(f"mid-bf16 class weights N={cfg.N} D={cfg.D} V={cfg.V}")
    gpu = run_gpu(case, "bf16", reduction="mean", chunk_rows=cfg.chunk_rows, class_weight=cw)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], None, case["t"], reduction="mean",
                                      class_weight=cw)
    errs = check_all(gpu, ref, "bf16", "mean", z=oracle.logits(case["X"], case["W"], None))
    log(f"mid-bf16 class weights errors {errs}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_unit_weights_are_bit_identical(dt):
    require_gpu()
    case = li.small_case(200, 64, 500, dtype=dt, seed=22, ignore_frac=0.1)
    for reduction in ("mean", "sum"):
        a = run_gpu(case, dt, reduction=reduction, chunk_rows=64)
        b = run_gpu(case, dt, reduction=reduction, chunk_rows=64,
                    class_weight=np.ones(500, np.float32))
        for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax", "n_valid"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"{reduction} {k}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_zero_total_weight(dt):
    """Every counted row's class weighs 0: the mean loss and every gradient
    are NaN (0/0 on the pages); the sum is 0 with zero gradients."""
    require_gpu()
    case = li.small_case(90, 32, 300, dtype=dt, seed=23, ignore_frac=0.2)
    cw = li.class_weights(300, seed=23)
    cw[case["t"][case["t"] >= 0]] = 0.0
    gm = run_gpu(case, dt, reduction="mean", chunk_rows=40, class_weight=cw)
    assert math.isnan(gm["loss"][0]) and int(gm["n_valid"][0]) == 72
    for k in ("grad_X", "grad_W", "grad_b"):
        assert np.all(np.isnan(gm[k])), k
    gs = run_gpu(case, dt, reduction="sum", chunk_rows=40, class_weight=cw)
    assert gs["loss"][0] == 0.0
    for k in ("grad_X", "grad_W", "grad_b"):
        assert np.all(gs[k] == 0.0), k


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_class_weights_with_ignore_index_in_range_and_bad_targets(dt):
    """ignore_index=7 is a class id; targets 300 and -5 are out of range: both
    kinds of row weigh 0 whatever class_weight holds."""
    require_gpu()
    case = li.small_case(150, 32, 300, dtype=dt, seed=24, ignore_frac=0.0)
    case["t"][[3, 40, 77]] = 7
    case["t"][[5, 90]] = 300
    case["t"][[6]] = -5
    cw = li.class_weights(300, seed=24)
    gpu = run_gpu(case, dt, reduction="mean", chunk_rows=64, ignore_index=7, class_weight=cw)
    ref = _ref(case, cw, "mean", ignore_index=7)
    check_all(gpu, ref, dt, "mean", z=_z(case))
    assert int(gpu["n_bad"][0]) == 3


@pytest.mark.parametrize("V", [1000, 32004, 100000])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_ce_inplace_class_weights(V, reduction):
    """Streamed rows (V up to 32004) and on-chip rows (V = 100000)."""
    require_gpu()
    rng = np.random.default_rng(V + 7)
    N = 61
    z = (rng.standard_normal((N, V)) * 3.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[[0, 30]] = -100
    cw = li.class_weights(V, seed=V, zero_frac=0.1)
    cw[t[5]] = 0.0
    log(f"ce class weights V={V} reduction={reduction}")
    loss, nv, dl = run_ce(z, t, reduction=reduction, grad_scale=1.5, class_weight=cw)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction, grad_scale=1.5,
                                                    class_weight=cw)
    assert nv == N - 2
    if reduction == "none":
        assert rel_err(loss, ref_loss) <= 1e-5
        assert loss[5] == 0.0
    else:
        assert abs(loss[0] - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(dl, ref_dl) <= 1e-4
    assert np.all(dl[[0, 5, 30]] == 0.0)
