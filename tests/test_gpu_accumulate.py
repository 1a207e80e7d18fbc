"""GPU parity of LCE_ACCUMULATE (gradients added into the caller's buffers,
beta = 1): every grad_W path (one group, several groups through the fp32
accumulator, compact, staged dL^T), grad_X's split sum, grad_b, the 'none'
backward, and an empty batch that must leave the buffers untouched.  The
expected value is the seeded prefill plus the oracle's gradient."""
import numpy as np
import pytest
import torch

import lce_inputs as li
from gpu_common import TOL, TORCH_DT, log, oracle, require_gpu
from linear_cross_entropy_chunk_amd import LinearCrossEntropy

pytestmark = pytest.mark.gpu


def _dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(TORCH_DT[dt])


def _prefill(shape, scale, dt, seed):
    a = (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)
    return li.round_to_bf16(a) if dt == "bf16" else (li.round_to_f16(a) if dt == "f16" else a)


def _check(got, pre, ref, dt, name):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - (pre.astype(np.float64) + ref)).max() / max(np.abs(ref).max(), 1e-30)
    # 16-bit types: one rounding of a sum about twice the gradient's size
    bound = TOL[dt]["grad"] * (1.0 if dt == "f32" else 2.0)
    assert err <= bound, f"{name} accumulate error {err:.3e}"


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("policy,chunk", [("accurate", 64), ("compact", 64), ("accurate", 0),
                                          ("accurate", -1)])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_accumulate_adds_into_existing_gradients(dt, policy, chunk, reduction):
    require_gpu()
    N, D, V = 300, 64, 777
    case = li.small_case(N, D, V, dtype=dt, seed=41, ignore_frac=0.1)
    up = case["u"] if reduction == "none" else None
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction=reduction, upstream=up)
    log(f"accumulate {dt} {policy} chunk={chunk} {reduction}")
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=True, reduction=reduction,
                            chunk_rows=chunk, acc_policy=policy, accumulate=True)
    pre = {k: _prefill(ref[k].shape, np.abs(ref[k]).max(), dt, seed)
           for seed, k in enumerate(("grad_X", "grad_W", "grad_b"))}
    out = {k: _dev(v, dt) for k, v in pre.items()}
    ud = None if up is None else torch.from_numpy(up.astype(np.float32)).to("cuda")
    op(_dev(case["X"], dt), _dev(case["W"], dt), torch.from_numpy(case["t"]).to("cuda"),
       _dev(case["b"], dt), grad_output=ud, out=out)
    torch.cuda.synchronize()
    for k in ("grad_X", "grad_W", "grad_b"):
        _check(out[k], pre[k], ref[k], dt, k)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_accumulate_twice_is_twice_the_gradient(dt):
    require_gpu()
    N, D, V = 200, 64, 500
    case = li.small_case(N, D, V, dtype=dt, seed=42, ignore_frac=0.1)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction="sum")
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=True, reduction="sum", chunk_rows=64,
                            accumulate=True)
    out = {"grad_X": torch.zeros(N, D, dtype=TORCH_DT[dt], device="cuda"),
           "grad_W": torch.zeros(V, D, dtype=TORCH_DT[dt], device="cuda"),
           "grad_b": torch.zeros(V, dtype=TORCH_DT[dt], device="cuda")}
    args = (_dev(case["X"], dt), _dev(case["W"], dt), torch.from_numpy(case["t"]).to("cuda"),
            _dev(case["b"], dt))
    op(*args, out=out)
    op(*args, out=out)
    torch.cuda.synchronize()
    for k in ("grad_X", "grad_W", "grad_b"):
        _check(out[k], np.zeros_like(ref[k]), 2.0 * ref[k], dt, k)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_accumulate_with_grad_x_stored_by_its_gemm(dt):
    """4096 rows x D=4096 form one grad_W group of four 1024-row chunks and
    256 grad_X tiles, so grad_X needs no K split and its GEMM adds into the
    caller's buffer itself (the fp16 path also unscales dL there)."""
    require_gpu()
    N, D, V = 4096, 4096, 512
    case = li.small_case(N, D, V, dtype=dt, seed=43, ignore_frac=0.05, bias=False)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], None, case["t"], reduction="mean")
    log(f"accumulate, grad_X stored by the GEMM, {dt}")
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], reduction="mean", chunk_rows=1024,
                            accumulate=True)
    pre = {k: _prefill(ref[k].shape, np.abs(ref[k]).max(), dt, seed)
           for seed, k in enumerate(("grad_X", "grad_W"))}
    out = {k: _dev(v, dt) for k, v in pre.items()}
    op(_dev(case["X"], dt), _dev(case["W"], dt), torch.from_numpy(case["t"]).to("cuda"),
       out=out)
    torch.cuda.synchronize()
    for k in ("grad_X", "grad_W"):
        _check(out[k], pre[k], ref[k], dt, k)


def test_accumulate_empty_batch_leaves_buffers():
    require_gpu()
    D, V = 32, 300
    op = LinearCrossEntropy(0, D, V, torch.float32, bias=True, reduction="sum", accumulate=True)
    gw = torch.full((V, D), 3.0, device="cuda")
    gb = torch.full((V,), -2.0, device="cuda")
    out = {"grad_X": torch.empty(0, D, device="cuda"), "grad_W": gw, "grad_b": gb}
    op(torch.empty(0, D, device="cuda"), torch.zeros(V, D, device="cuda"),
       torch.empty(0, dtype=torch.int64, device="cuda"), torch.zeros(V, device="cuda"), out=out)
    torch.cuda.synchronize()
    assert torch.all(gw == 3.0) and torch.all(gb == -2.0)


def test_accumulate_needs_the_buffers():
    require_gpu()
    op = LinearCrossEntropy(8, 32, 16, torch.float32, accumulate=True)
    x = torch.zeros(8, 32, device="cuda")
    with pytest.raises(ValueError):
        op(x, torch.zeros(16, 32, device="cuda"), torch.zeros(8, dtype=torch.int64,
                                                               device="cuda"))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_accumulate_with_ragged_groups(dt, reduction):
    """256-row chunks four to a group with a ragged end (N=1700: groups of
    1024 and 676 rows, the last chunk 164 rows), bias: the bf16 path sums
    grad_b once per group and forms grad_X once per group; every gradient
    adds into the caller's buffers."""
    require_gpu()
    N, D, V = 1700, 512, 3001
    case = li.small_case(N, D, V, dtype=dt, seed=44, ignore_frac=0.1)
    up = case["u"] if reduction == "none" else None
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction=reduction, upstream=up)
    log(f"accumulate, ragged groups, {dt} {reduction}")
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=True, reduction=reduction,
                            chunk_rows=256, accumulate=True)
    pre = {k: _prefill(ref[k].shape, np.abs(ref[k]).max(), dt, seed)
           for seed, k in enumerate(("grad_X", "grad_W", "grad_b"))}
    out = {k: _dev(v, dt) for k, v in pre.items()}
    ud = None if up is None else torch.from_numpy(up.astype(np.float32)).to("cuda")
    op(_dev(case["X"], dt), _dev(case["W"], dt), torch.from_numpy(case["t"]).to("cuda"),
       _dev(case["b"], dt), grad_output=ud, out=out)
    torch.cuda.synchronize()
    for k in ("grad_X", "grad_W", "grad_b"):
        _check(out[k], pre[k], ref[k], dt, k)
