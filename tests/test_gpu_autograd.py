"""GPU parity of the autograd entry points against the fp64 oracle: the
scalar reductions (gradients formed in the forward, scaled by the upstream
scalar in the backward), allow_retain_graph, the per-row 'none' op (recomputed
backward), requires_grad subsets, no_grad, batched input shapes, the
chunking options, higher-order derivatives refused, and the in-place
cross-entropy with mark_dirty."""
import numpy as np
import pytest
import torch

import lce_inputs as li
from gpu_common import OUT_ROUND, TOL, TORCH_DT, log, oracle, rel_err, require_gpu
from linear_cross_entropy_chunk_amd import LinearCrossEntropyOptions
from linear_cross_entropy_chunk_amd.functional import cross_entropy_inplace, linear_cross_entropy

pytestmark = pytest.mark.gpu


def _leaf(a, dt, grad=True):
    if a is None:
        return None
    x = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(TORCH_DT[dt])
    return x.requires_grad_(grad)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _case(dt, seed=31, N=300, D=64, V=777):
    case = li.small_case(N, D, V, dtype=dt, seed=seed, ignore_frac=0.1)
    cw = li.class_weights(V, seed=seed, zero_frac=0.05)
    return case, cw


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_scalar_backward_matches_oracle(dt, reduction):
    require_gpu()
    case, cw = _case(dt)
    X, W, b = _leaf(case["X"], dt), _leaf(case["W"], dt), _leaf(case["b"], dt)
    t = torch.from_numpy(case["t"]).to("cuda")
    cwd = torch.from_numpy(cw).to("cuda")
    log(f"autograd {reduction} {dt}")
    opts = LinearCrossEntropyOptions(batch_chunk_size=70, chunking_method=None)
    loss = linear_cross_entropy(X, W, t, b, weight=cwd, reduction=reduction, options=opts)
    assert loss.shape == () and loss.dtype == TORCH_DT[dt]
    (loss * 0.7).backward()
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction=reduction, grad_scale=0.7, class_weight=cw)
    tol = TOL[dt]
    assert abs(loss.item() - ref["loss"]) <= (tol["loss"] + OUT_ROUND[dt]) * abs(ref["loss"])
    # autograd hands the backward 0.7 rounded to the loss dtype, as for the pages' op
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction=reduction, class_weight=cw,
                                      grad_scale=float(torch.tensor(0.7, dtype=TORCH_DT[dt])))
    for got, key in ((X.grad, "grad_X"), (W.grad, "grad_W"), (b.grad, "grad_b")):
        assert got.dtype == TORCH_DT[dt]
        assert rel_err(_np(got), ref[key]) <= tol["grad"], key


def test_second_backward_raises_without_allow_retain_graph():
    require_gpu()
    case, _ = _case("f32")
    X, W = _leaf(case["X"], "f32"), _leaf(case["W"], "f32")
    t = torch.from_numpy(case["t"]).to("cuda")
    loss = linear_cross_entropy(X, W, t)
    loss.backward(retain_graph=True)
    with pytest.raises(RuntimeError, match="allow_retain_graph"):
        loss.backward()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_allow_retain_graph_backwards_twice(dt):
    require_gpu()
    case, cw = _case(dt, seed=32)
    X, W, b = _leaf(case["X"], dt), _leaf(case["W"], dt), _leaf(case["b"], dt)
    t = torch.from_numpy(case["t"]).to("cuda")
    opts = LinearCrossEntropyOptions(allow_retain_graph=True)
    loss = linear_cross_entropy(X, W, t, b, options=opts)
    loss.backward(retain_graph=True)
    g1 = [_np(p.grad) for p in (X, W, b)]
    (2.0 * loss).backward()
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"])
    for p, first, key in zip((X, W, b), g1, ("grad_X", "grad_W", "grad_b")):
        assert rel_err(first, ref[key]) <= TOL[dt]["grad"], key
        assert rel_err(_np(p.grad), 3.0 * ref[key]) <= TOL[dt]["grad"], key


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_none_reduction_recomputes_in_backward(dt):
    """(B, T, D) input, per-row loss of shape (B, T); the backward twice
    (retain_graph) gives twice the upstream-weighted gradients."""
    require_gpu()
    case, cw = _case(dt, seed=33, N=6 * 50)
    X = _leaf(case["X"].reshape(6, 50, -1), dt)
    W, b = _leaf(case["W"], dt), _leaf(case["b"], dt)
    t = torch.from_numpy(case["t"].reshape(6, 50)).to("cuda")
    cwd = torch.from_numpy(cw).to("cuda")
    u = case["u"].astype(np.float32)
    loss = linear_cross_entropy(X, W, t, b, weight=cwd, reduction="none")
    assert loss.shape == (6, 50) and loss.dtype == TORCH_DT[dt]
    ud = torch.from_numpy(u.reshape(6, 50)).to("cuda")
    (loss * ud).sum().backward(retain_graph=True)
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction="none", upstream=u, class_weight=cw)
    tol = TOL[dt]
    assert rel_err(_np(loss).reshape(-1), ref["loss"]) <= tol["loss"] + OUT_ROUND[dt]
    zero = ref["w"] == 0.0                  # ignored rows and zero-weight classes
    assert zero.any() and np.all(_np(loss).reshape(-1)[zero] == 0.0)
    assert rel_err(_np(X.grad).reshape(-1, X.shape[-1]), ref["grad_X"]) <= tol["grad"]
    assert rel_err(_np(W.grad), ref["grad_W"]) <= tol["grad"]
    assert rel_err(_np(b.grad), ref["grad_b"]) <= tol["grad"]
    (loss * ud).sum().backward()
    assert rel_err(_np(W.grad), 2.0 * ref["grad_W"]) <= tol["grad"]


def test_requires_grad_subsets_and_no_grad():
    require_gpu()
    case, _ = _case("f32", seed=34)
    t = torch.from_numpy(case["t"]).to("cuda")
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"])
    X, W, b = _leaf(case["X"], "f32"), _leaf(case["W"], "f32", False), _leaf(case["b"], "f32",
                                                                              False)
    linear_cross_entropy(X, W, t, b).backward()
    assert W.grad is None and b.grad is None
    assert rel_err(_np(X.grad), ref["grad_X"]) <= TOL["f32"]["grad"]
    X2, W2 = _leaf(case["X"], "f32", False), _leaf(case["W"], "f32")
    linear_cross_entropy(X2, W2, t, b).backward()
    assert X2.grad is None and rel_err(_np(W2.grad), ref["grad_W"]) <= TOL["f32"]["grad"]
    with torch.no_grad():
        loss = linear_cross_entropy(X, W2, t, b)
    assert not loss.requires_grad
    assert abs(loss.item() - ref["loss"]) <= TOL["f32"]["loss"] * abs(ref["loss"])


def test_higher_order_derivatives_are_refused():
    require_gpu()
    case, _ = _case("f32", seed=35)
    X, W = _leaf(case["X"], "f32"), _leaf(case["W"], "f32")
    t = torch.from_numpy(case["t"]).to("cuda")
    loss = linear_cross_entropy(X, W, t)
    (gx,) = torch.autograd.grad(loss, X, create_graph=True)
    with pytest.raises(RuntimeError):
        gx.sum().backward()


@pytest.mark.parametrize("method,bcs", [("auto", None), ("aspect_ratio:4", None), (None, 100),
                                        (None, None), ("aspect_ratio", 32)])
def test_chunking_options_give_the_same_result(method, bcs):
    """N=300, D=64, V=777: aspect_ratio plans next_pow2(ceil(300 / 13)) = 32
    rows, aspect_ratio:4 eight, None one chunk (the planned sizes are pinned
    in the CPU tests); every choice must give the oracle's gradients."""
    require_gpu()
    case, _ = _case("f32", seed=36)
    X, W = _leaf(case["X"], "f32"), _leaf(case["W"], "f32")
    t = torch.from_numpy(case["t"]).to("cuda")
    opts = LinearCrossEntropyOptions(chunking_method=method, batch_chunk_size=bcs,
                                     acc_policy="accurate")
    linear_cross_entropy(X, W, t, options=opts).backward()
    ref = oracle.linear_cross_entropy(case["X"], case["W"], None, case["t"])
    assert rel_err(_np(X.grad), ref["grad_X"]) <= TOL["f32"]["grad"]
    assert rel_err(_np(W.grad), ref["grad_W"]) <= TOL["f32"]["grad"]


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_inplace_cross_entropy_autograd(reduction):
    """logits = X W^T (fp32, X requires grad); the loss overwrites the logits
    with its gradient and the backward carries it into X.grad."""
    require_gpu()
    rng = np.random.default_rng(37)
    N, D, V = 96, 32, 1000
    Xn = rng.standard_normal((N, D)).astype(np.float32)
    Wn = (rng.standard_normal((V, D)) / np.sqrt(D)).astype(np.float32)
    tn = rng.integers(0, V, N)
    tn[[3, 40]] = -100
    cw = li.class_weights(V, seed=37)
    X = torch.from_numpy(Xn).to("cuda").requires_grad_(True)
    W = torch.from_numpy(Wn).to("cuda")
    logits = X @ W.T
    v0 = logits._version
    loss = cross_entropy_inplace(logits, torch.from_numpy(tn).to("cuda"),
                                 weight=torch.from_numpy(cw).to("cuda"), reduction=reduction)
    assert logits._version > v0
    u = rng.standard_normal(N).astype(np.float32)
    if reduction == "none":
        (loss * torch.from_numpy(u).to("cuda")).sum().backward()
    else:
        (1.5 * loss).backward()
    z = Xn.astype(np.float64) @ Wn.astype(np.float64).T
    ref_loss, dl = oracle.softmax_cross_entropy(z, tn, reduction=reduction, class_weight=cw,
                                                grad_scale=1.0)
    if reduction == "none":
        dl = dl * u[:, None]
        assert rel_err(_np(loss), ref_loss) <= 1e-5
    else:
        dl = 1.5 * dl
        assert abs(loss.item() - ref_loss) <= 1e-5 * abs(ref_loss)
    assert rel_err(_np(X.grad), dl @ Wn.astype(np.float64)) <= 1e-4


def test_inplace_cross_entropy_refuses_a_leaf():
    require_gpu()
    z = torch.zeros(4, 8, device="cuda", requires_grad=True)
    with pytest.raises(RuntimeError):
        cross_entropy_inplace(z, torch.zeros(4, dtype=torch.int64, device="cuda"))
