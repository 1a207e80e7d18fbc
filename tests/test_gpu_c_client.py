"""The C ABI from a plain C program (tests/c_abi/lce_client.c, built with
the library): no PyTorch in the process, only include/lce.h and the HIP
runtime for device memory.  Its outputs must match the fp64 oracle to the
dtype's tolerance and the Python binding's outputs bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import lce_inputs as li
from gpu_common import check_all, log, oracle, rel_err, require_gpu, run_ce, run_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_abi", "lce_client")
DTYPE = {"f32": (0, np.float32), "bf16": (1, None), "f16": (2, np.float16)}
REDUCTION = {"mean": 0, "sum": 1, "none": 2}


def _raw(a: np.ndarray, dt: str) -> bytes:
    """Elements of the input dtype; bf16 as the top half of fp32 (the values
    are exact bf16 already)."""
    a = np.ascontiguousarray(a, np.float32)
    if dt == "bf16":
        return (a.view(np.uint32) >> 16).astype(np.uint16).tobytes()
    return a.astype(DTYPE[dt][1]).tobytes()


def _decode(buf: bytes, n: int, dt: str) -> np.ndarray:
    if dt == "bf16":
        u = np.frombuffer(buf, np.uint16, n).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return np.frombuffer(buf, DTYPE[dt][1], n).astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_c_client_matches_oracle_and_binding(dt, reduction, tmp_path):
    require_gpu()
    assert os.path.exists(CLIENT), f"{CLIENT} is missing: run __graft_entry__.build()"
    N, D, V, chunk = 300, 64, 777, 64
    case = li.small_case(N, D, V, dtype=dt, seed=51, ignore_frac=0.1)
    hdr = np.array([N, D, V, chunk, DTYPE[dt][0], REDUCTION[reduction], 1], np.int64)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(hdr.tobytes())
        for a in (case["X"], case["W"], case["b"]):
            f.write(_raw(a, dt))
        f.write(np.ascontiguousarray(case["t"], np.int64).tobytes())
    log(f"C client {dt} {reduction}")
    r = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    buf = out.read_bytes()
    es = 4 if dt == "f32" else 2
    n_loss = N if reduction == "none" else 1
    o = 0
    got = {"loss": np.frombuffer(buf, np.float32, n_loss, o).astype(np.float64)}
    o += 4 * n_loss
    got["n_valid"] = np.frombuffer(buf, np.int64, 1, o)
    got["n_bad"] = np.frombuffer(buf, np.int64, 1, o + 8)
    o += 16
    for key, n in (("grad_X", N * D), ("grad_W", V * D), ("grad_b", V)):
        got[key] = _decode(buf[o:o + n * es], n, dt)
        o += n * es
    assert o == len(buf)
    got["grad_X"] = got["grad_X"].reshape(N, D)
    got["grad_W"] = got["grad_W"].reshape(V, D)

    # the 'none' backward with a unit upstream gradient on every row
    up = np.ones(N, np.float32) if reduction == "none" else None
    ref = oracle.linear_cross_entropy(case["X"], case["W"], case["b"], case["t"],
                                      reduction=reduction, upstream=up)
    check_all(got, ref, dt, reduction)
    py = run_gpu(case, dt, reduction=reduction, chunk_rows=chunk, argmax=False, upstream=up)
    for key in ("loss", "grad_X", "grad_W", "grad_b", "n_valid", "n_bad"):
        np.testing.assert_array_equal(got[key], py[key], err_msg=key)


@pytest.mark.parametrize("V", [1000, 100000])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_c_client_ce_inplace(V, reduction, tmp_path):
    """lce_ce_inplace from C: streamed rows (V = 1000) and on-chip rows
    (V = 100000)."""
    require_gpu()
    assert os.path.exists(CLIENT), f"{CLIENT} is missing: run __graft_entry__.build()"
    N = 37
    rng = np.random.default_rng(V + 52)
    z = (rng.standard_normal((N, V)) * 2.0).astype(np.float32)
    t = rng.integers(0, V, N).astype(np.int64)
    t[[0, 9]] = -100
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([N, V, REDUCTION[reduction]], np.int64).tobytes())
        f.write(z.tobytes())
        f.write(t.tobytes())
    log(f"C client ce V={V} {reduction}")
    r = subprocess.run([CLIENT, "ce", str(inp), str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    buf = out.read_bytes()
    n_loss = N if reduction == "none" else 1
    loss = np.frombuffer(buf, np.float32, n_loss, 0).astype(np.float64)
    nv = int(np.frombuffer(buf, np.int64, 1, 4 * n_loss)[0])
    dl = np.frombuffer(buf, np.float32, N * V, 4 * n_loss + 8).reshape(N, V).astype(np.float64)
    assert 4 * n_loss + 8 + 4 * N * V == len(buf)
    ref_loss, ref_dl = oracle.softmax_cross_entropy(z, t, reduction=reduction)
    assert nv == N - 2
    assert rel_err(loss, np.atleast_1d(ref_loss)) <= 1e-5
    assert rel_err(dl, ref_dl) <= 1e-4
    assert np.all(dl[[0, 9]] == 0.0)
    if reduction == "none":
        assert np.all(loss[[0, 9]] == 0.0)     # ignored rows: exactly 0
    py_loss, py_nv, py_dl = run_ce(z, t, reduction=reduction)
    np.testing.assert_array_equal(loss, py_loss)
    np.testing.assert_array_equal(dl, py_dl)
    assert nv == py_nv
