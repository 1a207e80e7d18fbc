"""The fused call and the standalone CE captured into a HIP graph (torch's
CUDAGraph over the HIP runtime) and replayed.  The library allocates nothing,
clears nothing with a memset and never synchronises inside a call, so one
call records as a plain chain of kernel nodes on the capturing stream.

Each replay is checked against an eager call on the same inputs, bit for bit
(both paths are deterministic), with eager work and synchronisations between
the replays: new inputs copied into the captured buffers and the outputs
poisoned with NaN, so a replay that skipped a kernel or read stale inputs
would show.  The first case is also checked against the oracle."""
import numpy as np
import pytest
import torch

import lce_inputs as li
from gpu_common import TORCH_DT, check_all, log, oracle, require_gpu, to_dev
from linear_cross_entropy_chunk_amd import CrossEntropyInplace, LinearCrossEntropy

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _host(out: dict) -> dict:
    return {k: v.detach().cpu().float().numpy() if v.is_floating_point() else v.cpu().numpy()
            for k, v in out.items()}


def _same(got: dict, want: dict, what: str) -> None:
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"{what}: {k}")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_fused_call_replays_from_a_graph(dt, reduction):
    """N=300 in 64-row chunks (a ragged last chunk), V=777 (a ragged last
    tile), bias, argmax, every gradient."""
    require_gpu()
    N, D, V = 300, 64, 777
    cases = [li.small_case(N, D, V, dtype=dt, seed=60 + k, ignore_frac=0.1)
             for k in range(REPLAYS)]
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=True, reduction=reduction,
                            chunk_rows=64, argmax=True)

    def upload(case):
        u = None
        if reduction == "none":
            u = torch.from_numpy(case["u"].astype(np.float32)).to("cuda")
        return (to_dev(case["X"], dt), to_dev(case["W"], dt),
                torch.from_numpy(case["t"]).to("cuda"), to_dev(case["b"], dt), u)

    # eager results, each call with its own outputs
    eager = []
    for case in cases:
        X, W, t, b, u = upload(case)
        eager.append(_host(op(X, W, t, b, grad_output=u)))
    torch.cuda.synchronize()

    # the buffers the graph is captured on
    X, W, t, b, u = upload(cases[0])
    out = op.make_outputs(grads=True)
    io = op.make_io(X, W, t, b, out=out, grad_output=u)
    op.run_io(io)                            # eager warm-up on the same buffers
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        op.run_io(io)
    log(f"graph {dt} {reduction}: captured")

    for k, case in enumerate(cases):
        Xk, Wk, tk, bk, uk = upload(case)
        X.copy_(Xk)
        W.copy_(Wk)
        t.copy_(tk)
        b.copy_(bk)
        if u is not None:
            u.copy_(uk)
        for v in out.values():
            if v.is_floating_point():
                v.fill_(float("nan"))
            else:
                v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _host(out)
        _same(got, eager[k], f"replay {k}")
        if k == 0:
            ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                              reduction=reduction, upstream=case["u"]
                                              if reduction == "none" else None)
            got64 = {kk: v.astype(np.float64) if v.dtype == np.float32 else v
                     for kk, v in got.items()}
            check_all(got64, ref, dt, reduction,
                      z=oracle.logits(case["X"], case["W"], case["b"]))
    del graph


@pytest.mark.parametrize("V", [1000, 8192, 50257, 100000, 160001])
def test_ce_inplace_replays_from_a_graph(V):
    """Every kernel of the standalone CE: one row per wave (V = 1000), on
    chip with 256 threads (8192), with rows at every alignment (50257) and
    aligned (100000), and two passes (160001); the logits are restored from
    a pristine copy before every replay."""
    require_gpu()
    N = 61
    rng = np.random.default_rng(V + 3)
    pristine = [torch.from_numpy((rng.standard_normal((N, V)) * 3.0).astype(np.float32))
                .to("cuda") for _ in range(REPLAYS)]
    targets = [torch.from_numpy(rng.integers(0, V, N)).to("cuda") for _ in range(REPLAYS)]
    for tt in targets:
        tt[[0, 30]] = -100
    op = CrossEntropyInplace(N, V, reduction="mean")
    eager = []
    for z0, tt in zip(pristine, targets):
        z = z0.clone()
        loss, nv = op(z, tt)
        eager.append({"dl": z.cpu().numpy(), "loss": loss.cpu().numpy(), "nv": nv.cpu().numpy()})
    torch.cuda.synchronize()

    z = pristine[0].clone()
    t = targets[0].clone()
    op(z, t)                                 # eager warm-up on the same buffers
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loss, nv = op(z, t)
    log(f"graph ce V={V}: captured")
    for k in range(REPLAYS):
        z.copy_(pristine[k])
        t.copy_(targets[k])
        loss.fill_(float("nan"))
        nv.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same({"dl": z.cpu().numpy(), "loss": loss.cpu().numpy(), "nv": nv.cpu().numpy()},
              eager[k], f"replay {k}")
    del graph


@pytest.mark.parametrize("chunk,group", [(64, 64), (256, 1024)])
def test_repair_replays_from_a_graph(chunk, group):
    """bf16 keeps one softmax reference per row and recomputes, behind a
    device-side flag, the chunks with a row whose loss exceeds 40 nats.  Three
    replays of one captured call: the second's inputs have two such rows
    (input rows scaled by 32, targets at their rows' lowest logits), so its
    gated repair launches recompute while the first's and third's do
    nothing.  Per-chunk combine (64-row chunks) and per-group combine
    (256-row chunks, four to a group); every replay bit for bit against an
    eager call, the far one also against the oracle."""
    require_gpu()
    N, D, V = 1024, 64, 2000
    far = [300, 700]

    def make(seed, with_far):
        case = li.small_case(N, D, V, dtype="bf16", seed=seed, ignore_frac=0.05)
        if with_far:
            X = case["X"].copy()
            X[far] *= 32.0
            z = oracle.logits(X, case["W"], case["b"])
            t = case["t"].copy()
            t[far] = np.argmin(z[far], axis=1)
            case = {**case, "X": X, "t": t}
        return case

    cases = [make(70, False), make(71, True), make(72, False)]
    op = LinearCrossEntropy(N, D, V, torch.bfloat16, bias=True, reduction="mean",
                            chunk_rows=chunk, argmax=True, group_rows=group)

    def upload(case):
        return (to_dev(case["X"], "bf16"), to_dev(case["W"], "bf16"),
                torch.from_numpy(case["t"]).to("cuda"), to_dev(case["b"], "bf16"))

    eager = []
    for case in cases:
        eager.append(_host(op(*upload(case))))
    torch.cuda.synchronize()

    X, W, t, b = upload(cases[0])
    out = op.make_outputs(grads=True)
    io = op.make_io(X, W, t, b, out=out)
    op.run_io(io)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        op.run_io(io)
    log(f"graph repair chunk={chunk} group={group}: captured")
    for k, case in enumerate(cases):
        Xk, Wk, tk, bk = upload(case)
        X.copy_(Xk)
        W.copy_(Wk)
        t.copy_(tk)
        b.copy_(bk)
        for v in out.values():
            if v.is_floating_point():
                v.fill_(float("nan"))
            else:
                v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _host(out)
        _same(got, eager[k], f"replay {k}")
        if k == 1:
            ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                              reduction="mean")
            got64 = {kk: v.astype(np.float64) if v.dtype == np.float32 else v
                     for kk, v in got.items()}
            check_all(got64, ref, "bf16", "mean",
                      z=oracle.logits(case["X"], case["W"], case["b"]))
    del graph
