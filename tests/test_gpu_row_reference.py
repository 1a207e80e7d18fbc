"""Rows far from their target.  The bf16 gradient path keeps one softmax
reference per row, its target logit: the chunk's tile holds exp(z - z_target)
and the gradient GEMMs apply g / S per row.  A row whose largest logit lies
more than 40 nats above its target logit (a loss above 40 nats) has its
256-row tile recomputed with the row max as reference.  These cases drive that recompute
(every row of every chunk; one row in one chunk of several, beside an ignored
row; every plan) and compare with the fp64 oracle, for bf16 and, on the same
inputs, for fp16 and fp32, whose path keeps per-block maxima."""
import numpy as np
import pytest

import lce_inputs as li
from gpu_common import check_all, log, oracle, require_gpu, run_gpu

pytestmark = pytest.mark.gpu

GAP = 40.0   # nats between the row max and the target logit that force the recompute


def _ref(case, reduction="mean", upstream=None):
    return oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                       reduction=reduction, upstream=upstream)


def _far_targets(case, rows):
    """Targets of `rows` set to their row's lowest logit (the largest loss)."""
    z = oracle.logits(case["X"], case["W"], case["b"])
    t = case["t"].copy()
    t[rows] = np.argmin(z[rows], axis=1)
    return {**case, "t": t}, z


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_every_row_far_from_its_target(dt):
    """Logits of spread ~12 per row and every target at the row minimum: almost
    every row's loss exceeds 40 nats, so every chunk is recomputed."""
    require_gpu()
    N, D, V = 300, 64, 1000
    case = li.small_case(N, D, V, dtype=dt, seed=81, ignore_frac=0.1, w_std=12.0 / np.sqrt(D))
    counted = np.nonzero(case["t"] != li.IGNORE_INDEX)[0]
    case, z = _far_targets(case, counted)
    gap = z.max(axis=1) - z[np.arange(N), np.where(case["t"] >= 0, case["t"], 0)]
    far = int((gap[counted] > GAP + 1.0).sum())
    assert far > counted.size // 2, far
    log(f"far rows dt={dt}: {far} of {counted.size} counted rows beyond {GAP} nats")
    gpu = run_gpu(case, dt, chunk_rows=64)
    check_all(gpu, _ref(case), dt, "mean", z=z)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("group_rows", [0, 128])
def test_one_far_row_in_one_chunk(dt, group_rows):
    """One row of chunk 2 (of 5) has its input scaled by 32 (exact in every
    dtype), so its logits spread ~32 and its loss is far above 40 nats; an
    ignored row sits in the same chunk.  Only that row's tile (the whole
    128-row chunk) is recomputed; the result matches the oracle and repeats
    bit for bit."""
    require_gpu()
    N, D, V = 600, 64, 2000
    case = li.small_case(N, D, V, dtype=dt, seed=82, ignore_frac=0.0)
    X = case["X"].copy()
    X[300] *= 32.0
    t = case["t"].copy()
    t[301] = li.IGNORE_INDEX
    case = {**case, "X": X, "t": t}
    case, z = _far_targets(case, [300])
    assert z[300].max() - z[300, case["t"][300]] > GAP + 1.0
    log(f"one far row dt={dt} group_rows={group_rows}")
    a, b = run_gpu(case, dt, chunk_rows=128, group_rows=group_rows, repeat=2)
    for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    check_all(a, _ref(case), dt, "mean", z=z)


@pytest.mark.parametrize("policy", ["accurate", "compact"])
def test_far_rows_with_none_reduction(policy):
    """'none' with an upstream gradient per row, far rows in two chunks, both
    grad_W policies."""
    require_gpu()
    N, D, V = 400, 64, 1500
    case = li.small_case(N, D, V, dtype="bf16", seed=83, ignore_frac=0.1)
    X = case["X"].copy()
    X[[10, 250]] *= 32.0
    case = {**case, "X": X}
    case, z = _far_targets(case, [10, 250])
    up = case["u"]
    gpu = run_gpu(case, "bf16", reduction="none", chunk_rows=128, upstream=up, acc_policy=policy)
    check_all(gpu, _ref(case, "none", up), "bf16", "none", z=z)


@pytest.mark.parametrize("far_rows", [[600], [5, 300, 700, 1000]])
def test_far_rows_with_the_combine_per_group(far_rows):
    """256-row chunks, four to a grad_W group: the statistics, the combine,
    the gated repair and the grad_b sums run once per group, the repair
    recomputing only the flagged 256-row tiles.  One far row in chunk 2, or
    one in every chunk; an ignored row beside the first."""
    require_gpu()
    N, D, V = 1024, 64, 2000
    case = li.small_case(N, D, V, dtype="bf16", seed=84, ignore_frac=0.05)
    X = case["X"].copy()
    X[far_rows] *= 32.0
    t = case["t"].copy()
    t[far_rows[0] + 1] = li.IGNORE_INDEX
    case = {**case, "X": X, "t": t}
    case, z = _far_targets(case, far_rows)
    assert all(z[r].max() - z[r, case["t"][r]] > GAP + 1.0 for r in far_rows)
    log(f"far rows per group: {far_rows}")
    a, b = run_gpu(case, "bf16", chunk_rows=256, group_rows=1024, repeat=2)
    for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    check_all(a, _ref(case), "bf16", "mean", z=z)


def test_combine_per_group_matches_per_chunk():
    """The same problem with the combine per group (256-row chunks) and per
    chunk (group_rows = the chunk rows): both meet the oracle's bar, and their
    losses agree to fp32 rounding."""
    require_gpu()
    N, D, V = 1024, 64, 3000
    case = li.small_case(N, D, V, dtype="bf16", seed=85, ignore_frac=0.1)
    grp = run_gpu(case, "bf16", chunk_rows=256, group_rows=1024)
    per = run_gpu(case, "bf16", chunk_rows=256, group_rows=256)
    ref = _ref(case)
    check_all(grp, ref, "bf16", "mean")
    check_all(per, ref, "bf16", "mean")
    assert abs(grp["loss"][0] - per["loss"][0]) <= 1e-6 * abs(ref["loss"])


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_loss_only_forward_with_the_combine_per_group(dt):
    """'none' without an upstream gradient (the loss-only forward) with
    256-row chunks four to a group: the statistics of the group's chunks
    are combined once, after its last chunk; a ragged last group (three
    chunks, the last one short).  Per-row loss and argmax against the
    oracle, and the per-chunk combine gives the same losses."""
    require_gpu()
    N, D, V = 1700, 64, 2500
    case = li.small_case(N, D, V, dtype=dt, seed=86, ignore_frac=0.1)
    grp = run_gpu(case, dt, reduction="none", chunk_rows=256, group_rows=1024)
    per = run_gpu(case, dt, reduction="none", chunk_rows=256, group_rows=256)
    ref = _ref(case, "none")
    check_all(grp, ref, dt, "none", z=oracle.logits(case["X"], case["W"], case["b"]), grads="")
    np.testing.assert_allclose(grp["loss"], per["loss"], rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(grp["argmax"], per["argmax"])


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("group_rows", [0, 768])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ragged_groups_with_gradients(dt, group_rows, reduction):
    """Gradients with 256-row chunks several to a group and a ragged end:
    N=1700 in 256-row chunks (the last one 164 rows), D=512, V=3001 (a
    ragged last class tile), bias, 10% ignored rows.  The default cap holds
    1024 rows for 16-bit types (groups of 4 chunks and 3: 256, 256, 164
    rows) and 512 for fp32 (groups of 2, the last one 164 rows); a cap of
    768 rows gives groups of 3 chunks, the last one a single short chunk.
    bf16 combines each group once after its last chunk; every dtype keeps
    group-sized statistics.  'none' runs the backward with an upstream
    gradient per row."""
    require_gpu()
    N, D, V = 1700, 512, 3001
    case = li.small_case(N, D, V, dtype=dt, seed=87, ignore_frac=0.1)
    up = case["u"] if reduction == "none" else None
    log(f"ragged groups dt={dt} group_rows={group_rows} {reduction}")
    gpu = run_gpu(case, dt, reduction=reduction, chunk_rows=256, group_rows=group_rows,
                  upstream=up)
    check_all(gpu, _ref(case, reduction, up), dt, reduction,
              z=oracle.logits(case["X"], case["W"], case["b"]))


def test_far_rows_in_a_ragged_last_group():
    """The gated repair in a ragged last group: N=1700 in 256-row chunks,
    four to a group (1024 and 676 rows), far rows in the second group's
    first chunk and in its last chunk of 164 rows, beside an ignored row."""
    require_gpu()
    N, D, V = 1700, 64, 2000
    far = [1100, 1650]
    case = li.small_case(N, D, V, dtype="bf16", seed=88, ignore_frac=0.05)
    X = case["X"].copy()
    X[far] *= 32.0
    t = case["t"].copy()
    t[1651] = li.IGNORE_INDEX
    case = {**case, "X": X, "t": t}
    case, z = _far_targets(case, far)
    assert all(z[r].max() - z[r, case["t"][r]] > GAP + 1.0 for r in far)
    log("far rows in a ragged last group")
    for reduction in ("mean", "none"):
        up = case["u"] if reduction == "none" else None
        gpu = run_gpu(case, "bf16", reduction=reduction, chunk_rows=256, group_rows=1024,
                      upstream=up)
        check_all(gpu, _ref(case, reduction, up), "bf16", reduction, z=z)


@pytest.mark.parametrize("group_rows", [1024, 2048])
def test_far_row_inside_a_long_chunk(group_rows):
    """1024-row chunks (four 256-row tiles each), one far row in the third
    tile of the second chunk and one in the last tile of the last chunk:
    only those tiles' rows are recomputed, per chunk (group_rows = the chunk)
    or per group of two chunks."""
    require_gpu()
    N, D, V = 3000, 64, 2500
    far = [1024 + 600, 2990]
    case = li.small_case(N, D, V, dtype="bf16", seed=89, ignore_frac=0.05)
    X = case["X"].copy()
    X[far] *= 32.0
    case = {**case, "X": X}
    case, z = _far_targets(case, far)
    assert all(z[r].max() - z[r, case["t"][r]] > GAP + 1.0 for r in far)
    log(f"far rows inside long chunks, group_rows={group_rows}")
    a, b = run_gpu(case, "bf16", chunk_rows=1024, group_rows=group_rows, repeat=2)
    for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    check_all(a, _ref(case), "bf16", "mean", z=z)


@pytest.mark.parametrize("chunk", [64, 128, 192])
def test_far_rows_with_short_chunks_sharing_a_launch(chunk):
    """Chunks shorter than a 256-row tile, several to a group: the group's
    chunks share one logits launch and one combine, and the gated repair
    recomputes the 256-row tiles of the far rows (which straddle chunk
    boundaries).  N=1000 with groups of 512 rows (a ragged last group)."""
    require_gpu()
    N, D, V = 1000, 64, 1800
    far = [100, 700, 990]
    case = li.small_case(N, D, V, dtype="bf16", seed=90, ignore_frac=0.05)
    X = case["X"].copy()
    X[far] *= 32.0
    case = {**case, "X": X}
    case, z = _far_targets(case, far)
    log(f"far rows, {chunk}-row chunks sharing a launch")
    a, b = run_gpu(case, "bf16", chunk_rows=chunk, group_rows=512, repeat=2)
    for k in ("loss", "grad_X", "grad_W", "grad_b", "argmax"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    check_all(a, _ref(case), "bf16", "mean", z=z)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_loss_only_forward_with_short_chunks_sharing_a_launch(dt):
    """'none' without an upstream gradient in 64-row chunks, eight to a
    group: one logits launch and one combine per group; the per-chunk plan
    gives the same losses."""
    require_gpu()
    N, D, V = 1100, 64, 2500
    case = li.small_case(N, D, V, dtype=dt, seed=91, ignore_frac=0.1)
    grp = run_gpu(case, dt, reduction="none", chunk_rows=64, group_rows=512)
    per = run_gpu(case, dt, reduction="none", chunk_rows=64, group_rows=64)
    ref = _ref(case, "none")
    check_all(grp, ref, dt, "none", z=oracle.logits(case["X"], case["W"], case["b"]), grads="")
    np.testing.assert_allclose(grp["loss"], per["loss"], rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(grp["argmax"], per["argmax"])
