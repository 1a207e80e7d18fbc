"""The timing hook of the C ABI (lce_timing_enable / lce_timing_read), which
the benchmark's per-kernel times and roofline come from: one timed launch
per kernel launch of a selected class, and a read that fails loudly when
launches found the event pool full instead of returning partial totals as
whole ones."""
import numpy as np
import pytest
import torch

import lce_inputs as li
from gpu_common import TORCH_DT, log, require_gpu, to_dev
from linear_cross_entropy_chunk_amd import LinearCrossEntropy
from linear_cross_entropy_chunk_amd import _binding as B

pytestmark = pytest.mark.gpu

ALL = (1 << B.LCE_K_COUNT) - 1


def _op_and_args(N, chunk, group_rows=0):
    case = li.small_case(N, 64, 1000, dtype="bf16", seed=111, ignore_frac=0.1)
    op = LinearCrossEntropy(N, 64, 1000, TORCH_DT["bf16"], bias=True, reduction="mean",
                            chunk_rows=chunk, group_rows=group_rows)
    args = (to_dev(case["X"], "bf16"), to_dev(case["W"], "bf16"),
            torch.from_numpy(case["t"]).to("cuda"), to_dev(case["b"], "bf16"))
    return op, args


@pytest.mark.parametrize("chunk,group_rows,launches", [(256, 0, 3), (64, 512, 2)])
def test_one_timed_launch_per_logits_launch(chunk, group_rows, launches):
    """N=600 in 256-row chunks: one logits launch per chunk, 3 per call.  In
    64-row chunks eight to a group (groups of 512 and 88 rows), each group's
    chunks share one logits launch, as a 256-row tile would be mostly empty
    per chunk: 2 per call."""
    require_gpu()
    op, args = _op_and_args(600, chunk, group_rows)
    B.lce_timing_enable(op.handle, ALL)
    try:
        for _ in range(3):
            op(*args)
        torch.cuda.synchronize()
        t = B.lce_timing_read(op.handle)
    finally:
        B.lce_timing_enable(op.handle, 0)
    ms, n = t["logits"]
    assert n == 3 * launches and ms > 0.0
    assert t["gemm_x"][1] >= 3 and t["gemm_w"][1] >= 3
    log(f"timed classes: { {k: v for k, v in t.items() if v[1]} }")


def test_pool_overflow_is_reported():
    """One-row chunks (256 per call, several timed launches each): enough
    calls to pass the pool's 4096 pairs.  The read returns UNSUPPORTED with
    the count of untimed launches; the pool then starts over, and a read
    within it succeeds."""
    require_gpu()
    op, args = _op_and_args(256, 1)
    B.lce_timing_enable(op.handle, ALL)
    try:
        for _ in range(8):
            op(*args)
        torch.cuda.synchronize()
        with pytest.raises(B.LceError) as err:
            B.lce_timing_read(op.handle)
        assert err.value.status == B.LCE_ERR_UNSUPPORTED
        assert "not timed" in str(err.value)
        op(*args)
        torch.cuda.synchronize()
        t = B.lce_timing_read(op.handle)
        assert t["logits"][1] == 256
    finally:
        B.lce_timing_enable(op.handle, 0)
