"""grad_W's last round split along K.  When the D/256 x V/256 output tiles
leave a partial last round of at most half the CUs, the trailing 256-class
tile columns that hold it run as a second launch with K split into fp32
partials, summed into grad_W's last rows.  D = 512 and V = 35840 give 2 x 140
tiles, 24 past the last full round: 12 tile columns, 4 K ranges over the
1024-row chunk.  V = 35740 gives the same tiles with a ragged last column
(156 classes), so the split starts at a tile boundary 2972 classes before V.
Checked against the fp64 oracle for every element type (fp32 reads the
staged dL^T, the 16-bit types T's panels), both policies, several chunks per
call, 'none', and adding into existing gradients."""
import numpy as np
import pytest
import torch

import lce_inputs as li
from gpu_common import TOL, TORCH_DT, check_all, log, oracle, require_gpu, run_gpu
from linear_cross_entropy_chunk_amd import LinearCrossEntropy

pytestmark = pytest.mark.gpu

N, D, V = 1024, 512, 35840
V_RAGGED = 35740        # 140 tile columns, the last one 156 classes


def _ref(case, reduction="mean", upstream=None):
    return oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                       reduction=reduction, upstream=upstream)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("policy", ["accurate", "compact"])
@pytest.mark.parametrize("v", [V, V_RAGGED])
def test_tail_columns_split_along_k(dt, policy, v):
    require_gpu()
    case = li.small_case(N, D, v, dtype=dt, seed=91, ignore_frac=0.05)
    log(f"grad_W tail split dt={dt} {policy} V={v}")
    gpu = run_gpu(case, dt, chunk_rows=N, acc_policy=policy)
    ref_w = _ref(case)["grad_W"]
    check_all(gpu, _ref(case), dt, "mean",
              z=oracle.logits(case["X"], case["W"], case["b"]))
    # the split rows (the last 12 tile columns) are held to the same bar as the rest
    tail = slice(128 * 256, v)
    err = np.abs(gpu["grad_W"][tail] - ref_w[tail]).max() / np.abs(ref_w).max()
    assert err <= TOL[dt]["grad"], err


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_tail_split_with_a_ragged_last_column_over_several_chunks(dt):
    """compact, 512-row chunks: each chunk's grad_W launch splits its tail
    (K = 512 in 2 ranges) and adds it into the 16-bit grad_W, with the
    ragged last tile column."""
    require_gpu()
    case = li.small_case(1500, D, V_RAGGED, dtype=dt, seed=95, ignore_frac=0.05)
    log(f"grad_W tail split, compact over chunks, ragged V, {dt}")
    gpu = run_gpu(case, dt, chunk_rows=512, acc_policy="compact")
    check_all(gpu, _ref(case), dt, "mean", z=oracle.logits(case["X"], case["W"], case["b"]))


def test_tail_split_with_none_reduction():
    require_gpu()
    case = li.small_case(N, D, V, dtype="bf16", seed=92, ignore_frac=0.0)
    up = case["u"]
    gpu = run_gpu(case, "bf16", reduction="none", chunk_rows=N, upstream=up)
    check_all(gpu, _ref(case, "none", up), "bf16", "none")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_tail_split_adds_into_existing_gradients(dt):
    """LCE_ACCUMULATE: the split sum adds into grad_W's last rows as the main
    launch's epilogue adds into the others."""
    require_gpu()
    case = li.small_case(N, D, V, dtype=dt, seed=93, ignore_frac=0.05)
    ref = _ref(case)
    rng = np.random.default_rng(94)
    pre = (rng.standard_normal((V, D)) * np.abs(ref["grad_W"]).max()).astype(np.float32)
    pre = li.round_to_bf16(pre) if dt == "bf16" else pre
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=True, reduction="mean",
                            chunk_rows=N, grad_x=False, grad_b=False, accumulate=True)
    out = {"grad_W": torch.from_numpy(pre).to("cuda").to(TORCH_DT[dt])}
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(TORCH_DT[dt])
    op(dev(case["X"]), dev(case["W"]), torch.from_numpy(case["t"]).to("cuda"), dev(case["b"]),
       out=out)
    torch.cuda.synchronize()
    got = out["grad_W"].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - (pre.astype(np.float64) + ref["grad_W"])).max() / np.abs(ref["grad_W"]).max()
    assert err <= TOL[dt]["grad"] * (1.0 if dt == "f32" else 2.0), err
