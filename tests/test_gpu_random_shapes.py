"""GPU parity on seeded random shapes: rows, features, classes, chunk sizes,
dtype, reduction, bias, accumulation policy and the share of ignored rows are
drawn per case, so combinations the hand-picked cases miss (ragged chunks
inside grad_W groups, groups of one, K split or not, tiles mostly empty) meet
the oracle.  The draws are fixed by the case index; each case prints its
parameters before it runs."""
import numpy as np
import pytest

import lce_inputs as li
from gpu_common import check_all, log, oracle, require_gpu, run_gpu

pytestmark = pytest.mark.gpu

CASES = 24


def _params(i: int) -> dict:
    rng = np.random.default_rng([2024, i])
    dt = ["f32", "bf16", "f16"][i % 3]
    vec = 4 if dt == "f32" else 8
    N = int(rng.integers(1, 900))
    p = {
        "dt": dt,
        "N": N,
        "D": int(vec * rng.integers(1, 80)),
        "V": int(rng.integers(1, 3000)),
        "chunk": int(rng.choice([0, -1, int(rng.integers(1, N + 1)), 64, 128])),
        "reduction": str(rng.choice(["mean", "sum", "none"])),
        "bias": bool(rng.integers(0, 2)),
        "policy": str(rng.choice(["accurate", "compact"])),
        "ignore": float(rng.choice([0.0, 0.1, 0.5])),
    }
    return p


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    require_gpu()
    p = _params(i)
    log(f"random case {i}: {p}")
    case = li.small_case(p["N"], p["D"], p["V"], dtype=p["dt"], bias=p["bias"],
                         ignore_frac=p["ignore"], seed=100 + i)
    up = case["u"] if p["reduction"] == "none" else None
    gpu = run_gpu(case, p["dt"], reduction=p["reduction"], chunk_rows=p["chunk"],
                  acc_policy=p["policy"], upstream=up, bias=p["bias"])
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"] if p["bias"] else None,
                                      case["t"], reduction=p["reduction"], upstream=up)
    z = oracle.logits(case["X"], case["W"], case["b"] if p["bias"] else None)
    if p["reduction"] == "mean" and ref["n_valid"] == 0:
        assert np.isnan(gpu["loss"][0])
        return
    errs = check_all(gpu, ref, p["dt"], p["reduction"], z=z,
                     grads="xwb" if p["bias"] else "xw")
    log(f"random case {i} errors {errs}")
