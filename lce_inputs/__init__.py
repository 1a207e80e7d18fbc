"""Seeded synthetic inputs for the chunked linear-cross-entropy workloads.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic, so both the fp64 oracle and the GPU path may use it.

Every large tensor is drawn in row blocks, block ``k`` of tensor ``key`` from
its own stream ``numpy.random.default_rng([seed, key, k])``.  The values are
therefore fixed by (seed, key, block size) alone, blocks can be drawn in
parallel threads, and any block can be redrawn on its own.

Stream keys: 0 X, 1 W, 2 b, 3 targets, 4 ignore-row permutation,
5 upstream per-row gradient, 6 standalone-CE logits, 7 per-class weights.

bf16 and fp16 tensors are returned as float32 arrays whose values are
exactly representable in that type (rounded to nearest-even from the float32
draw), so a ``torch.tensor(...).to(torch.bfloat16)`` (or float16) upload is
exact and an upcast to float64 on the CPU is exact as well.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100

KEY_X, KEY_W, KEY_B, KEY_T, KEY_IGN, KEY_U, KEY_LOGITS, KEY_CW = range(8)

# Elements per generator block (rows per block = BLOCK_ELEMS // row_length).
BLOCK_ELEMS = 1 << 22


@dataclasses.dataclass(frozen=True)
class LceConfig:
    """One fused linear-cross-entropy workload."""
    name: str
    N: int
    D: int
    V: int
    dtype: str                  # "f32", "bf16" or "f16"
    has_bias: bool
    targets: str                # "uniform" or "zipf1.1"
    ignore_frac: float          # exact count = round(frac * N) rows
    reduction: str              # "mean", "sum" or "none"
    chunk_rows: int             # 0 = aspect-ratio heuristic
    seed: int = 0
    upstream: bool = False      # 'none' backward: per-row upstream grad ~ N(0,1)


@dataclasses.dataclass(frozen=True)
class CeConfig:
    """Standalone softmax cross-entropy on precomputed fp32 logits."""
    name: str
    N: int
    V: int
    reduction: str
    seed: int = 0


# The five workloads.  Readings of the distributions: N(0, s) is read as
# variance s (so W ~ N(0, 1/D) has std 1/sqrt(D) and b ~ N(0, 0.01) has
# std 0.1); seed 0 for every workload.
TINY_F32 = LceConfig("tiny-f32", 256, 64, 1000, "f32", True, "uniform", 0.10,
                     "mean", 64)
MID_BF16 = LceConfig("mid-bf16", 4096, 2048, 32000, "bf16", False, "uniform",
                     0.05, "mean", 1024)
LARGE_VOCAB_BF16 = LceConfig("large-vocab-bf16", 8192, 4096, 128256, "bf16",
                             False, "zipf1.1", 0.05, "mean", 2048)
NONE_BF16 = LceConfig("none-bf16", 16384, 4096, 151936, "bf16", True,
                      "uniform", 0.0, "none", 0, upstream=True)
CE_F32 = CeConfig("ce-f32", 16384, 131072, "mean")

LCE_CONFIGS = {c.name: c for c in (TINY_F32, MID_BF16, LARGE_VOCAB_BF16, NONE_BF16)}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 holding bf16-exact values.  Inputs here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def round_to_f16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest IEEE binary16 value (ties to even),
    returned as float32.  Inputs here are finite and far inside fp16's range."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


def _round(vals: np.ndarray, rounding) -> np.ndarray:
    """rounding: True or "bf16", "f16", or False / None / "f32" (none)."""
    if rounding is True or rounding == "bf16":
        return round_to_bf16(vals)
    if rounding == "f16":
        return round_to_f16(vals)
    return vals


def _rows_per_block(row_len: int) -> int:
    return max(1, BLOCK_ELEMS // max(1, row_len))


def normal_rows(rows: int, cols: int, std: float, seed: int, key: int,
                bf16, row_start: int = 0, row_stop: int | None = None
                ) -> np.ndarray:
    """Rows [row_start, row_stop) of a (rows, cols) float32 N(0, std^2) draw,
    rounded per ``bf16`` (True or "bf16", "f16", or False for none).

    The draw is defined block by block, so a row range gives the same values
    as the corresponding slice of the full tensor."""
    if row_stop is None:
        row_stop = rows
    rpb = _rows_per_block(cols)
    out = np.empty((row_stop - row_start, cols), dtype=np.float32)
    first_blk = row_start // rpb
    last_blk = (row_stop - 1) // rpb if row_stop > row_start else first_blk - 1

    def fill(blk: int) -> None:
        b0 = blk * rpb
        b1 = min(rows, b0 + rpb)
        rng = np.random.default_rng([seed, key, blk])
        vals = rng.standard_normal((b1 - b0) * cols, dtype=np.float32)
        vals = vals.reshape(b1 - b0, cols)
        vals *= np.float32(std)
        vals = _round(vals, bf16)
        s0, s1 = max(b0, row_start), min(b1, row_stop)
        out[s0 - row_start:s1 - row_start] = vals[s0 - b0:s1 - b0]

    blocks = range(first_blk, last_blk + 1)
    if len(blocks) <= 1:
        for b in blocks:
            fill(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    return out


def zipf_ranks(n: int, V: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Draw n ranks in [0, V) with P(k) proportional to (k+1)^-s, k = 0..V-1,
    by inverse transform of the truncated distribution's CDF."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    k = np.searchsorted(cdf, u, side="right")
    return np.minimum(k, V - 1).astype(np.int64)


def targets(N: int, V: int, dist: str, ignore_frac: float, seed: int,
            ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """int64 class targets; exactly round(ignore_frac * N) rows, chosen by a
    seeded permutation, are set to ignore_index."""
    rng = np.random.default_rng([seed, KEY_T, 0])
    if dist == "uniform":
        t = rng.integers(0, V, size=N, dtype=np.int64)
    elif dist.startswith("zipf"):
        t = zipf_ranks(N, V, float(dist[4:]), rng)
    else:
        raise ValueError(f"unknown target distribution {dist!r}")
    n_ign = int(round(ignore_frac * N))
    if n_ign:
        perm = np.random.default_rng([seed, KEY_IGN, 0]).permutation(N)
        t[perm[:n_ign]] = ignore_index
    return t


def upstream_grad(N: int, seed: int) -> np.ndarray:
    """Per-row upstream gradient for reduction='none' backward, N(0,1) fp32."""
    return np.random.default_rng([seed, KEY_U, 0]).standard_normal(
        N, dtype=np.float32)


def class_weights(V: int, seed: int, zero_frac: float = 0.0) -> np.ndarray:
    """Per-class weights, float32 uniform in [0.25, 2); a ``zero_frac``
    share of the classes (a seeded choice) gets weight 0."""
    rng = np.random.default_rng([seed, KEY_CW, 0])
    w = rng.uniform(0.25, 2.0, V).astype(np.float32)
    n0 = int(round(zero_frac * V))
    if n0:
        w[rng.permutation(V)[:n0]] = 0.0
    return w


def lce_inputs(cfg: LceConfig, rows: slice | None = None) -> dict:
    """All inputs of a fused workload as numpy arrays.

    X, W, b are float32 arrays (exact in cfg.dtype when it is 'bf16' or 'f16');
    b is None without bias; t is int64; u (the per-row upstream gradient) is
    None unless cfg.upstream.  With ``rows`` only those rows of X, t and u are
    returned."""
    bf16 = cfg.dtype
    r0 = 0 if rows is None else (rows.start or 0)
    r1 = cfg.N if rows is None else (cfg.N if rows.stop is None else rows.stop)
    X = normal_rows(cfg.N, cfg.D, 1.0, cfg.seed, KEY_X, bf16, r0, r1)
    W = normal_rows(cfg.V, cfg.D, 1.0 / np.sqrt(cfg.D), cfg.seed, KEY_W, bf16)
    b = None
    if cfg.has_bias:
        b = normal_rows(1, cfg.V, 0.1, cfg.seed, KEY_B, bf16)[0]
    t = targets(cfg.N, cfg.V, cfg.targets, cfg.ignore_frac, cfg.seed)[r0:r1]
    u = upstream_grad(cfg.N, cfg.seed)[r0:r1] if cfg.upstream else None
    return {"X": X, "W": W, "b": b, "t": t, "u": u}


def ce_inputs(cfg: CeConfig, rows: slice | None = None) -> dict:
    """Standalone CE inputs: float32 logits ~ N(0,1) and uniform targets."""
    r0 = 0 if rows is None else (rows.start or 0)
    r1 = cfg.N if rows is None else (cfg.N if rows.stop is None else rows.stop)
    z = normal_rows(cfg.N, cfg.V, 1.0, cfg.seed, KEY_LOGITS, False, r0, r1)
    t = targets(cfg.N, cfg.V, "uniform", 0.0, cfg.seed)[r0:r1]
    return {"logits": z, "t": t}


def small_case(N: int, D: int, V: int, *, dtype: str = "f32", bias: bool = True,
               ignore_frac: float = 0.1, seed: int = 0, x_std: float = 1.0,
               w_std: float | None = None, dist: str = "uniform",
               ignore_index: int = IGNORE_INDEX) -> dict:
    """A small ad-hoc case with the same recipe as the named workloads; dtype
    'f32', 'bf16' or 'f16' fixes the rounding of X, W and b."""
    bf16 = dtype
    w_std = 1.0 / np.sqrt(max(D, 1)) if w_std is None else w_std
    X = normal_rows(N, D, x_std, seed, KEY_X, bf16) if N else np.zeros((0, D), np.float32)
    W = normal_rows(V, D, w_std, seed, KEY_W, bf16)
    b = normal_rows(1, V, 0.1, seed, KEY_B, bf16)[0] if bias else None
    t = targets(N, V, dist, ignore_frac, seed, ignore_index) if N else np.zeros(0, np.int64)
    u = upstream_grad(N, seed) if N else np.zeros(0, np.float32)
    return {"X": X, "W": W, "b": b, "t": t, "u": u}
