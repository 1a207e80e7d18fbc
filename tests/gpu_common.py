"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the fp64 oracle to the stated
tolerances.

Tolerances (one per input dtype; bf16 and fp16 inputs accumulate in fp32):
  loss            |dL| / |L|                      f32 1e-5   bf16 5e-3   f16 1e-4
  per-row loss    max |d loss_n| / max |loss_n|   f32 1e-5   bf16 5e-3   f16 1e-4
  each gradient   max |dG| / max |G_ref|          f32 1e-4   bf16 2e-2   f16 5e-3
fp16 (not among the stated bars) is derived from its unit roundoff 2^-11:
the loss comes from fp32 logits of exact inputs (rounding error ~1e-6, 1e-4
leaves a wide margin); a gradient carries one fp16 rounding of dL and one of
the output, together at most ~2 x 2^-11 ~ 1e-3 of max|G| when the target
term dominates a row, so 5e-3 is about five times that bound.
  n_valid, n_bad  bit-exact
  zero-weight rows (ignored, out-of-range target, class weight 0): per-row
                  loss ('none') and grad_X row bit-exact 0
  argmax          bit-exact where the oracle's top-2 gap exceeds
                  1e-4 * max(1, |row max|); elsewhere the GPU's class must
                  lie within that margin of the row max (a valid near-tie).
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from linear_cross_entropy_chunk_amd import CrossEntropyInplace, LinearCrossEntropy

TOL = {"f32": {"loss": 1e-5, "grad": 1e-4}, "bf16": {"loss": 5e-3, "grad": 2e-2},
       "f16": {"loss": 1e-4, "grad": 5e-3}}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# Unit roundoff of each input dtype: the autograd entry point returns the
# loss in the input dtype (the module source's output contract), one rounding
# of the fp32 loss, so its loss checks add this to the loss tolerance.
OUT_ROUND = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
ARGMAX_MARGIN = 1e-4


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu() -> None:
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"


def to_dev(a, dt: str):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(TORCH_DT[dt])


def run_gpu(case: dict, dt: str, *, reduction: str = "mean", chunk_rows: int = 0,
            acc_policy: str = "accurate", ignore_index: int = -100, grads: str = "xwb",
            argmax: bool = True, upstream=None, grad_scale: float = 1.0, bias: bool | None = None,
            repeat: int = 1, class_weight=None, group_rows: int = 0) -> dict | list:
    X, W, b, t = case["X"], case["W"], case["b"], case["t"]
    if bias is False:
        b = None
    N, D = X.shape
    V = W.shape[0]
    op = LinearCrossEntropy(N, D, V, TORCH_DT[dt], bias=b is not None, reduction=reduction,
                            ignore_index=ignore_index, chunk_rows=chunk_rows,
                            acc_policy=acc_policy, grad_x="x" in grads, grad_w="w" in grads,
                            grad_b=("b" in grads) and b is not None, argmax=argmax,
                            group_rows=group_rows)
    Xd, Wd, bd = to_dev(X, dt), to_dev(W, dt), to_dev(b, dt)
    td = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int64)).to("cuda")
    ud = None if upstream is None else torch.from_numpy(
        np.ascontiguousarray(upstream, dtype=np.float32)).to("cuda")
    cwd = None if class_weight is None else torch.from_numpy(
        np.ascontiguousarray(class_weight, dtype=np.float32)).to("cuda")
    results = []
    for _ in range(repeat):
        out = op(Xd, Wd, td, bd, grad_output=ud, grad_scale=grad_scale, class_weight=cwd)
        torch.cuda.synchronize()
        res = {}
        for k, v in out.items():
            res[k] = v.cpu().numpy() if v.dtype in (torch.int32, torch.int64) else \
                v.float().cpu().numpy().astype(np.float64)
        res["chunk_rows"] = op.chunk_rows
        res["ws_bytes"] = op.ws_bytes
        results.append(res)
    return results[0] if repeat == 1 else results


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def check_loss(got, ref, dt: str, reduction: str) -> float:
    if reduction == "none":
        e = rel_err(got, ref)
    else:
        got, ref = float(np.asarray(got).reshape(-1)[0]), float(ref)
        e = abs(got - ref) / max(abs(ref), 1e-6)
    assert e <= TOL[dt]["loss"], f"loss error {e:.3e} > {TOL[dt]['loss']}"
    return e


def check_grad(got, ref, dt: str, name: str) -> float:
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    e = rel_err(got, ref)
    assert e <= TOL[dt]["grad"], f"{name} error {e:.3e} > {TOL[dt]['grad']}"
    return e


def check_argmax(got, ref, gap, rowmax, z_at_got) -> int:
    """Exact where the oracle's top-2 gap is clear; a valid near-max class
    elsewhere.  Returns the number of near-tie rows."""
    margin = ARGMAX_MARGIN * np.maximum(1.0, np.abs(rowmax))
    clear = gap > margin
    bad = np.nonzero(clear & (got != ref))[0]
    assert bad.size == 0, f"argmax differs on clear rows {bad[:10]}"
    near = ~clear
    if near.any():
        assert np.all(z_at_got[near] >= rowmax[near] - margin[near])
    return int(near.sum())


def check_zero_rows(gpu: dict, ref: dict, reduction: str) -> int:
    """Rows that weigh nothing (ignored, target out of range, or a class of
    weight 0) give a per-row loss of exactly 0 ('none') and, where the row
    weight g is exactly 0, a grad_X row of exactly 0: bit-exact, not within a
    tolerance.  Returns the number of such rows."""
    w = np.asarray(ref["w"])
    zero = w == 0.0
    if reduction == "none" and "loss" in gpu:
        bad = np.nonzero(zero & (np.asarray(gpu["loss"]) != 0.0))[0]
        assert bad.size == 0, f"per-row loss not exactly 0 on zero-weight rows {bad[:10]}"
    if "grad_X" in gpu and gpu["grad_X"].shape[0]:
        gz = np.asarray(ref["g"]) == 0.0
        bad = np.nonzero(gz & np.any(gpu["grad_X"] != 0.0, axis=1))[0]
        assert bad.size == 0, f"grad_X row not exactly 0 on rows of weight 0 {bad[:10]}"
    return int(zero.sum())


def check_all(gpu: dict, ref: dict, dt: str, reduction: str, z=None, grads="xwb") -> dict:
    errs = {"loss": check_loss(gpu["loss"], ref["loss"], dt, reduction)}
    assert int(gpu["n_valid"][0]) == ref["n_valid"]
    assert int(gpu["n_bad"][0]) == ref["n_bad"]
    if "w" in ref:
        errs["zero_rows"] = check_zero_rows(gpu, ref, reduction)
    for key, flag in (("grad_X", "x"), ("grad_W", "w"), ("grad_b", "b")):
        if key in gpu and flag in grads:
            errs[key] = check_grad(gpu[key], ref[key], dt, key)
    if "argmax" in gpu and z is not None and z.shape[0]:
        zs = np.sort(z, axis=1)
        gap = zs[:, -1] - zs[:, -2] if z.shape[1] > 1 else np.full(z.shape[0], np.inf)
        z_at = z[np.arange(z.shape[0]), gpu["argmax"]]
        check_argmax(gpu["argmax"], ref["argmax"], gap, zs[:, -1], z_at)
    return errs


def run_ce(z: np.ndarray, t: np.ndarray, *, reduction: str = "mean", ignore_index: int = -100,
           grad_scale: float = 1.0, class_weight=None, offset: int = 0):
    """The standalone CE on a copy of z; with `offset` the logits start that
    many floats into a fresh allocation (4-byte, not 16-byte, alignment)."""
    flat = torch.empty(z.size + offset, dtype=torch.float32, device="cuda")
    zd = flat[offset:].view(z.shape)
    zd.copy_(torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)))
    td = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int64)).to("cuda")
    op = CrossEntropyInplace(z.shape[0], z.shape[1], reduction=reduction,
                             ignore_index=ignore_index)
    cwd = None if class_weight is None else torch.from_numpy(
        np.ascontiguousarray(class_weight, dtype=np.float32)).to("cuda")
    loss, nv = op(zd, td, grad_scale, cwd)
    torch.cuda.synchronize()
    return (loss.cpu().numpy().astype(np.float64), int(nv.cpu()[0]),
            zd.cpu().numpy().astype(np.float64))


__all__ = ["TOL", "log", "require_gpu", "run_gpu", "check_all", "check_loss", "check_grad",
           "check_argmax", "check_zero_rows", "rel_err", "run_ce", "oracle"]
