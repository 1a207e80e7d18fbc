"""GPU parity on seeded random shapes: rows, features, classes, chunk sizes,
dtype, reduction, bias, accumulation policy and the share of ignored rows are
drawn per case, so combinations the hand-picked cases miss (ragged chunks
inside grad_W groups, groups of one, K split or not, tiles mostly empty) meet
the oracle.  The draws are fixed by the case index; each case prints its
parameters before it runs.  A second set also draws the rows of dL per grad_W
GEMM, the requested gradients, class weights, the argmax, grad_scale and rows
far from their target; a third draws larger shapes whose grad_W output tiles
leave a partial last round held by trailing tile columns with a ragged last
one (V not a multiple of 256), the shapes whose tail is split along K."""
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


# Broader draws: every plan parameter varies, including how many rows of dL a
# grad_W GEMM holds (group_rows), which gradients are requested, per-class
# weights, the argmax, grad_scale, and rows whose loss exceeds 40 nats (input
# row scaled by 32, which forces the bf16 path's recompute).

def _plan_params(i: int, large: bool = False) -> dict:
    rng = np.random.default_rng([2025, i, int(large)])
    dt = ["f32", "bf16", "f16"][i % 3]
    vec = 4 if dt == "f32" else 8
    if large:
        # D and V drawn until grad_W's output tiles leave a partial last round
        # of at most 128 of the 256 CUs held by whole trailing tile columns,
        # the last of them ragged (V not a multiple of 256): the shapes whose
        # trailing columns are split along K
        for _ in range(10000):
            N = int(rng.integers(1024, 4097))
            D = int(vec * rng.integers(512 // vec, 1024 // vec + 1))
            V = int(rng.integers(9000, 30000))
            tm, tn = -(-D // 256), -(-V // 256)
            rem = (tm * tn) % 256
            cols = -(-rem // tm) if rem else 0
            if V % 256 and 0 < cols < tn and cols * tm <= 128:
                break
        else:
            raise AssertionError("no shape with a split tail drawn")
    else:
        N = int(rng.integers(1, 1500))
        D = int(vec * rng.integers(1, 80))
        V = int(rng.choice([int(rng.integers(1, 3000)), 256 * int(rng.integers(1, 12))]))
    chunk = int(rng.choice([0, -1, int(rng.integers(1, N + 1)), 128, 256, 512]))
    if large:   # grad_W over K of at least 512 rows, so that the tail is split
        chunk = int(rng.choice([0, -1, 512, 1024, int(rng.integers(512, N + 1))]))
    return {
        "dt": dt, "N": N, "D": D, "V": V, "chunk": chunk,
        "group_rows": int(rng.choice([0, 1, max(chunk, 1), 3 * max(chunk, 1), 1 << 20])),
        "reduction": str(rng.choice(["mean", "sum", "none"])),
        "upstream": bool(rng.integers(0, 4) > 0),
        "bias": bool(rng.integers(0, 2)),
        "policy": str(rng.choice(["accurate", "compact"])),
        "grads": str(rng.choice(["xwb", "xw", "w", "wb"] if large else
                                ["xwb", "xwb", "xw", "x", "w", "b", ""])),
        "argmax": bool(rng.integers(0, 2)),
        "ignore": float(rng.choice([0.0, 0.05, 0.3])),
        "class_weight": bool(rng.integers(0, 4) == 0),
        "far": int(rng.choice([0, 0, 1, 3])),
        "grad_scale": float(rng.choice([1.0, 0.5, 3.0])),
    }


def _run_plan(i: int, p: dict) -> None:
    case = li.small_case(p["N"], p["D"], p["V"], dtype=p["dt"], bias=p["bias"],
                         ignore_frac=p["ignore"], seed=300 + i)
    if p["far"]:
        rows = np.random.default_rng([2026, i]).choice(p["N"], size=min(p["far"], p["N"]),
                                                       replace=False)
        X = case["X"].copy()
        X[rows] *= 32.0
        case = {**case, "X": X}
    cw = None
    if p["class_weight"]:
        cw = np.random.default_rng([2027, i]).uniform(0.0, 2.0, p["V"]).astype(np.float32)
        cw[::7] = 0.0
    b = case["b"] if p["bias"] else None
    red = p["reduction"]
    up = case["u"] if red == "none" and p["upstream"] else None
    grads = p["grads"] if red != "none" or up is not None else ""
    grads = grads if p["bias"] else grads.replace("b", "")
    gs = p["grad_scale"] if red != "none" else 1.0
    gpu = run_gpu(case, p["dt"], reduction=red, chunk_rows=p["chunk"], acc_policy=p["policy"],
                  upstream=up, bias=p["bias"], grads=grads, argmax=p["argmax"], class_weight=cw,
                  group_rows=p["group_rows"], grad_scale=gs)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], b, case["t"], reduction=red,
                                      upstream=up, class_weight=cw, grad_scale=gs)
    if red == "mean" and not np.isfinite(ref["loss"]):      # no weight counted
        assert np.isnan(gpu["loss"][0])
        return
    z = oracle.logits(case["X"], case["W"], b) if p["argmax"] else None
    errs = check_all(gpu, ref, p["dt"], red, z=z, grads=grads)
    log(f"plan case {i} errors {errs}")


@pytest.mark.parametrize("i", range(32))
def test_random_plan(i):
    require_gpu()
    p = _plan_params(i)
    log(f"plan case {i}: {p}")
    _run_plan(i, p)


@pytest.mark.parametrize("i", range(6))
def test_random_large_shape_with_a_split_tail(i):
    require_gpu()
    p = _plan_params(i, large=True)
    log(f"large plan case {i}: {p}")
    _run_plan(100 + i, p)
