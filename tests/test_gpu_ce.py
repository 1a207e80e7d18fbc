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


@pytest.mark.parametrize("V", [65536, 100000, 131068, 131072, 151936])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ce_long_rows_on_chip(V, reduction):
    """Rows of 64K..152K classes take the single-read path (the row held in
    registers and LDS; 151936 classes with 1024 threads); ragged lengths
    exercise its partial vectors."""
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


def _check_ce(z, t, reduction, offset=0, grad_scale=1.0):
    loss, nv, dl = run_ce(z, t, reduction=reduction, offset=offset, grad_scale=grad_scale)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction,
                                                    grad_scale=grad_scale)
    ign = t == -100
    assert nv == int((~ign).sum())
    if reduction == "none":
        assert rel_err(loss, ref_loss) <= 1e-5
        assert np.all(loss[ign] == 0.0)
    else:
        assert abs(loss[0] - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(dl, ref_dl) <= 1e-4
    assert np.all(dl[ign] == 0.0)
    return dl


@pytest.mark.parametrize("V", [1, 2, 3, 5, 7, 1021, 2049, 4097, 8193, 16641, 50257])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ce_any_row_length(V, reduction):
    """V not a multiple of 4: row n starts n V mod 4 floats past a 16-byte
    boundary, so consecutive rows take every alignment, with their first and
    last elements outside the 16-byte vectors.  Targets on those elements
    (the first and last classes) and ignored rows included."""
    require_gpu()
    rng = np.random.default_rng(1000 + V)
    N = 13
    z = (rng.standard_normal((N, V)) * 3.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[[1, 2]] = [0, V - 1]
    t[5] = -100
    log(f"ce any length V={V} reduction={reduction}")
    _check_ce(z, t, reduction, grad_scale=1.25)


@pytest.mark.parametrize("V", [32004, 65537, 131071, 131073, 140001, 160001])
def test_ce_long_rows_not_a_multiple_of_4(V):
    """Rows that stay on chip (24K to 150K classes: registers, then the LDS
    tail; 512 threads up to 131072 classes, 1024 above) with consecutive
    rows at every alignment, and a row too long for the chip (160001
    classes), which streams twice."""
    require_gpu()
    rng = np.random.default_rng(V)
    N = 6
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[[0, 1]] = [V - 1, 0]
    t[3] = -100
    log(f"ce long unaligned rows V={V}")
    _check_ce(z, t, "none")


@pytest.mark.parametrize("V", [4096, 12000, 131072])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_ce_logits_off_a_16_byte_boundary(V, offset):
    """Logits that start 4, 8 or 12 bytes past a 16-byte boundary (a view into
    a larger buffer): accepted, and every row takes the element-wise head and
    tail, one row per wave (4096 classes) and on chip (12000 with 256
    threads, 131072 with 512)."""
    require_gpu()
    rng = np.random.default_rng(V + offset)
    N = 5
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    t = rng.integers(0, V, N)
    t[0] = V - 1
    t[2] = -100
    log(f"ce offset {offset} V={V}")
    _check_ce(z, t, "mean", offset=offset)


@pytest.mark.parametrize("V", [4096, 8193, 50257, 100000, 151936, 160001])
def test_ce_masked_logits(V):
    """Classes masked to -inf: the upper half of every row (whole threads'
    shares of the two-pass kernel, 160001 classes, see only -inf; 4096
    classes go one row per wave, 8193 to 151936 stay on chip), and all but
    three classes of one row.
    The loss stays finite and the masked gradient is exactly 0, as in the
    oracle (pinned to torch)."""
    require_gpu()
    rng = np.random.default_rng(2000 + V)
    N = 7
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    z[:, V // 2:] = -np.inf
    z[3, 3:] = -np.inf
    t = rng.integers(0, V // 2, N)
    t[3] = 1
    t[5] = -100
    log(f"ce masked V={V}")
    dl = _check_ce(z, t, "none")
    assert np.all(dl[:, V // 2:] == 0.0) and np.all(dl[3, 3:] == 0.0)
