"""The allocation-free standalone cross-entropy, lce_ce_inplace_noalloc,
through the C ABI.  It runs the kernels of lce_ce_inplace on a static device
scratch instead of a caller's workspace, so on the same inputs its loss,
n_valid and in-place gradient must equal lce_ce_inplace's bit for bit (and
meet the oracle's fp32 tolerances).  Two calls in a row, the second on a
smaller input, since every call on a GPU reuses the same scratch.  Sizes
beyond the scratch are refused on the host."""
import numpy as np
import pytest

from linear_cross_entropy_chunk_amd import _binding as B

REDUCTION = {"mean": B.LCE_MEAN, "sum": B.LCE_SUM, "none": B.LCE_NONE}

# (N, V, reduction, class weights): the first call on-chip rows, the second
# a smaller problem, one row per wave.
CALLS = [(300, 131072, "mean", False), (37, 1000, "none", True)]


def _inputs(N, V, weighted, seed):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    t = rng.integers(0, V, N).astype(np.int64)
    t[[0, N // 2]] = -100
    cw = rng.uniform(0.25, 2.0, V).astype(np.float32) if weighted else None
    return z, t, cw


def _call(entry, z, t, cw, reduction, grad_scale):
    import torch
    dev = torch.device("cuda", 0)
    N, V = z.shape
    zd = torch.from_numpy(z).to(dev)
    td = torch.from_numpy(t).to(dev)
    cwd = None if cw is None else torch.from_numpy(cw).to(dev)
    loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    cwp = None if cwd is None else cwd.data_ptr()
    if entry == "noalloc":
        B.lce_ce_inplace_noalloc(zd.data_ptr(), td.data_ptr(), cwp, N, V, -100,
                                 REDUCTION[reduction], grad_scale, loss.data_ptr(),
                                 nv.data_ptr(), stream)
    else:
        ws = torch.empty(B.lce_ce_workspace_size(N, V), dtype=torch.uint8, device=dev)
        B.lce_ce_inplace(zd.data_ptr(), td.data_ptr(), cwp, N, V, -100, REDUCTION[reduction],
                         grad_scale, loss.data_ptr(), nv.data_ptr(), ws.data_ptr(), ws.numel(),
                         stream)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), int(nv.cpu()[0]), zd.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_ce_matches_the_workspace_entry_point():
    import torch

    from gpu_common import log, oracle, rel_err, require_gpu
    require_gpu()
    for i, (N, V, reduction, weighted) in enumerate(CALLS):
        log(f"no-alloc CE call {i}: N={N} V={V} {reduction} weighted={weighted}")
        z, t, cw = _inputs(N, V, weighted, seed=70 + i)
        got = _call("noalloc", z, t, cw, reduction, 0.75)
        ref = _call("workspace", z, t, cw, reduction, 0.75)
        np.testing.assert_array_equal(got[0], ref[0])
        assert got[1] == ref[1] == N - 2
        np.testing.assert_array_equal(got[2], ref[2])
        o_loss, o_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction, grad_scale=0.75,
                                                    class_weight=cw)
        assert rel_err(got[0], np.atleast_1d(o_loss)) <= 1e-5
        assert rel_err(got[2], o_dl) <= 1e-4
        assert np.all(got[2][[0, N // 2]] == 0.0)
        if reduction == "none":
            assert np.all(got[0][[0, N // 2]] == 0.0)
    torch.cuda.empty_cache()


def test_noalloc_ce_refuses_more_rows_than_its_scratch():
    """N above LCE_CE_NOALLOC_MAX_ROWS returns UNSUPPORTED on the host, before
    anything is enqueued (the pointers are never dereferenced)."""
    fake = 1 << 20
    st = B.lce_ce_inplace_noalloc_status(fake, fake, B.LCE_CE_NOALLOC_MAX_ROWS + 1, 1024,
                                         B.LCE_MEAN, fake)
    assert st == B.LCE_ERR_UNSUPPORTED
    assert "exceeds the static scratch" in B.lce_last_error()
    assert B.lce_ce_inplace_noalloc_status(fake + 2, fake, 16, 1024, B.LCE_MEAN, fake) == \
        B.LCE_ERR_UNSUPPORTED                                  # logits not 4-byte aligned
    assert B.lce_ce_inplace_noalloc_status(fake, fake, 16, 1024, 7, fake) == \
        B.LCE_ERR_UNSUPPORTED                                  # unknown reduction
    assert B.lce_ce_inplace_noalloc_status(fake, fake, 16, 1024, B.LCE_MEAN, 0) == \
        B.LCE_ERR_INVALID_ARG                                  # no loss buffer


@pytest.mark.gpu
def test_noalloc_ce_replays_from_a_graph():
    """Captured into a HIP graph (the callers it is for), after one eager call
    on the device: each replay on new logits equals an eager call bit for
    bit, with eager work and synchronisations between the replays."""
    import torch

    from gpu_common import log, require_gpu
    require_gpu()
    dev = torch.device("cuda", 0)
    N, V = 64, 4096
    z, t, _ = _inputs(N, V, False, seed=80)
    zd = torch.from_numpy(z).to(dev)
    td = torch.from_numpy(t).to(dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int64, device=dev)

    def call():
        B.lce_ce_inplace_noalloc(zd.data_ptr(), td.data_ptr(), None, N, V, -100, B.LCE_MEAN,
                                 1.0, loss.data_ptr(), nv.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)

    call()                                    # eager: the scratch address is looked up here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    zd.copy_(torch.from_numpy(z).to(dev))
    with torch.cuda.graph(graph):
        call()
    log("no-alloc CE graph captured")
    for k in range(3):
        zk, tk, _ = _inputs(N, V, False, seed=81 + k)
        want = _call("noalloc", zk, tk, None, "mean", 1.0)      # eager, own buffers
        zd.copy_(torch.from_numpy(zk).to(dev))
        td.copy_(torch.from_numpy(tk).to(dev))
        loss.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(loss.cpu().numpy(), want[0])
        assert int(nv.cpu()[0]) == want[1]
        np.testing.assert_array_equal(zd.cpu().numpy(), want[2])
