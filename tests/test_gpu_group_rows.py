"""group_rows: how many chunks' dL one grad_W GEMM consumes (lce_desc).  On
small ragged shapes with several groups: one chunk per group (the per-chunk
path, fp32 accumulator across chunks), the default cap, three chunks per
group, and every chunk in one group, with 64-row-aligned chunks (dL read in
place from T) and unaligned ones (dL^T staged).  Each setting meets the
oracle's tolerance; groups that cover every row plan exactly as the default
when the default covers them too; results are deterministic."""
import numpy as np
import pytest

import lce_inputs as li
from gpu_common import check_all, log, oracle, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


def _ref(case, reduction="mean", upstream=None):
    return oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                       reduction=reduction, upstream=upstream)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("chunk", [128, 100])
@pytest.mark.parametrize("group_rows", [1, 0, 384, 1 << 20])
def test_group_rows_meet_the_oracle(dt, chunk, group_rows):
    """N=1100 in chunks of 128 (9 chunks, a 76-row tail) or 100 (11 chunks),
    D=128 (default cap 256 rows: 2 chunks of 128 per group), V=3001, bias,
    10% ignored rows, mean."""
    require_gpu()
    case = li.small_case(1100, 128, 3001, dtype=dt, seed=71, ignore_frac=0.1)
    log(f"group_rows={group_rows} chunk={chunk} dt={dt}")
    gpu = run_gpu(case, dt, chunk_rows=chunk, group_rows=group_rows)
    z = oracle.logits(case["X"], case["W"], case["b"])
    errs = check_all(gpu, _ref(case), dt, "mean", z=z)
    log(f"group_rows={group_rows} chunk={chunk} dt={dt} errors {errs}")


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_group_rows_other_reductions(reduction):
    require_gpu()
    case = li.small_case(900, 64, 2000, dtype="bf16", seed=72, ignore_frac=0.1)
    up = case["u"] if reduction == "none" else None
    for gr in (1, 0):
        gpu = run_gpu(case, "bf16", reduction=reduction, chunk_rows=128, upstream=up,
                      group_rows=gr)
        check_all(gpu, _ref(case, reduction, up), "bf16", reduction,
                  z=oracle.logits(case["X"], case["W"], case["b"]))


def test_group_rows_plans_and_determinism():
    """A cap at or above every row plans exactly as the default when the
    default already holds every row (same workspace, bit-identical results);
    one chunk per group needs the fp32 accumulator; runs repeat bit for
    bit."""
    require_gpu()
    case = li.small_case(512, 256, 1500, dtype="bf16", seed=73, ignore_frac=0.1)
    # default cap: 4 * 256 / 2 = 512 rows = every row (4 chunks of 128)
    a = run_gpu(case, "bf16", chunk_rows=128, group_rows=0)
    b = run_gpu(case, "bf16", chunk_rows=128, group_rows=512)
    c1, c2 = run_gpu(case, "bf16", chunk_rows=128, group_rows=128, repeat=2)
    assert a["ws_bytes"] == b["ws_bytes"]
    for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        np.testing.assert_array_equal(c1[k], c2[k], err_msg=k)
    assert c1["ws_bytes"] >= 1500 * 256 * 4          # the fp32 V x D accumulator
    ref = _ref(case)
    check_all(c1, ref, "bf16", "mean")
    check_all(a, ref, "bf16", "mean")
