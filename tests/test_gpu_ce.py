"""GPU parity of the standalone in-place softmax cross-entropy against the
fp64 oracle (fp32 logits, fp32 tolerances)."""
import math

import numpy as np
import pytest

from gpu_common import log, oracle, rel_err, require_gpu, run_ce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V", [4, 1000, 4096, 32004])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_ce_inplace_matches_oracle(V, reduction):
    require_gpu()
    rng = np.random.default_rng(V)
    N = 97
    z = (rng.standard_normal((N, V)) * 3.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[[0, 50]] = -100
    log(f"ce V={V} reduction={reduction}")
    loss, nv, dl = run_ce(z, t, reduction=reduction, grad_scale=1.5)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction, grad_scale=1.5)
    assert nv == N - 2
    if reduction == "none":
        assert rel_err(loss, ref_loss) <= 1e-5
        assert np.all(loss[[0, 50]] == 0.0)      # ignored rows: exactly 0
    else:
        assert abs(loss[0] - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(dl, ref_dl) <= 1e-4
    assert np.all(dl[[0, 50]] == 0.0)


def test_ce_large_logits_and_all_ignored():
    require_gpu()
    rng = np.random.default_rng(1)
    z = (rng.standard_normal((16, 2048)) * 50.0).astype(np.float32)
    t = rng.integers(0, 2048, 16)
    loss, _, dl = run_ce(z, t)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t)
    assert abs(loss[0] - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(dl, ref_dl) <= 1e-4
    t_all = np.full(16, -100)
    loss, nv, dl = run_ce(z, t_all)
    assert nv == 0 and math.isnan(loss[0]) and np.all(np.isnan(dl))


@pytest.mark.parametrize("V", [65536, 100000, 131068, 131072])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ce_long_rows_on_chip(V, reduction):
    """Rows of 64K..128K classes take the single-read path (the row held in
    registers and LDS); ragged lengths exercise its partial vectors."""
    require_gpu()
    rng = np.random.default_rng(V + 1)
    N = 9
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[4] = -100
    t[0] = V - 1                      # the last class, inside the LDS tail
    log(f"ce on-chip V={V} reduction={reduction}")
    loss, nv, dl = run_ce(z, t, reduction=reduction)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction)
    assert nv == N - 1
    if reduction == "none":
        assert rel_err(loss, ref_loss) <= 1e-5
        assert loss[4] == 0.0                    # the ignored row: exactly 0
    else:
        assert abs(loss[0] - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(dl, ref_dl) <= 1e-4
    assert np.all(dl[4] == 0.0)
