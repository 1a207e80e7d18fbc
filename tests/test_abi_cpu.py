"""The C ABI on the host (no GPU): the library loads, exports every function
include/lce.h declares, its structs have the layout ctypes assumes, and the
host-only entry points (validation, chunk planning, workspace sizing, status
strings) behave as documented.  No compute call is made."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_cross_entropy_chunk_amd as lce
from linear_cross_entropy_chunk_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from linear_cross_entropy_chunk_amd import build
        build.build(verbose=False)
    return B.lib()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LCE_API\s+[\w\s\*]+?\b(lce_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(lce_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_c(tmp_path):
    """Compile a probe against lce.h with the host C compiler and compare
    sizeof / offsetof with the ctypes mirrors."""
    src = tmp_path / "layout.c"
    fields_desc = [f[0] for f in B.lce_desc._fields_]
    fields_io = [f[0] for f in B.lce_io._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lce.h"', "int main(void) {",
             'printf("desc %zu\\n", sizeof(lce_desc));', 'printf("io %zu\\n", sizeof(lce_io));']
    lines += [f'printf("desc.{f} %zu\\n", offsetof(lce_desc, {f}));' for f in fields_desc]
    lines += [f'printf("io.{f} %zu\\n", offsetof(lce_io, {f}));' for f in fields_io]
    lines += ["return 0; }"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    assert int(got["desc"]) == ctypes.sizeof(B.lce_desc)
    assert int(got["io"]) == ctypes.sizeof(B.lce_io)
    for f in fields_desc:
        assert int(got[f"desc.{f}"]) == getattr(B.lce_desc, f).offset, f
    for f in fields_io:
        assert int(got[f"io.{f}"]) == getattr(B.lce_io, f).offset, f


def _desc(**kw):
    d = dict(N=256, D=64, V=1000, ignore_index=-100, chunk_rows=64, dtype=B.LCE_F32,
             acc_dtype=B.LCE_F32, has_bias=1, reduction=B.LCE_MEAN, acc_policy=B.LCE_ACCURATE,
             flags=B.LCE_GRAD_X | B.LCE_GRAD_W | B.LCE_GRAD_B)
    d.update(kw)
    return B.lce_desc(**d)


@pytest.mark.parametrize("kw,status", [
    ({}, B.LCE_OK),
    ({"N": -1}, B.LCE_ERR_INVALID_ARG),
    ({"D": 0}, B.LCE_ERR_INVALID_ARG),
    ({"V": 0}, B.LCE_ERR_INVALID_ARG),
    ({"chunk_rows": -2}, B.LCE_ERR_INVALID_ARG),
    ({"dtype": 7}, B.LCE_ERR_DTYPE),
    ({"acc_dtype": B.LCE_BF16}, B.LCE_ERR_UNSUPPORTED),           # fp32 input, bf16 acc
    ({"dtype": B.LCE_BF16, "acc_dtype": B.LCE_BF16}, B.LCE_OK),   # non-mixed
    ({"dtype": B.LCE_F16, "acc_dtype": B.LCE_F16}, B.LCE_OK),
    ({"dtype": B.LCE_BF16, "acc_dtype": B.LCE_F16}, B.LCE_ERR_UNSUPPORTED),
    ({"dtype": B.LCE_BF16, "acc_dtype": 7}, B.LCE_ERR_UNSUPPORTED),
    ({"reduction": 3}, B.LCE_ERR_UNSUPPORTED),          # the pages' NotImplementedError
    ({"acc_policy": 2}, B.LCE_ERR_INVALID_ARG),
    ({"has_bias": 0}, B.LCE_ERR_INVALID_ARG),            # grad_b requested without bias
    ({"flags": 32}, B.LCE_ERR_INVALID_ARG),
    ({"flags": B.LCE_GRAD_X | B.LCE_ACCUMULATE}, B.LCE_OK),
    ({"D": 62}, B.LCE_ERR_UNSUPPORTED),                  # fp32 rows not 16-byte aligned
    ({"dtype": B.LCE_BF16, "D": 60}, B.LCE_ERR_UNSUPPORTED),
    ({"dtype": B.LCE_BF16, "D": 64}, B.LCE_OK),
    ({"N": 0}, B.LCE_OK),
    ({"N": 1 << 32}, B.LCE_ERR_UNSUPPORTED),
    # 32-bit offsets inside a 256-row operand tile: row lengths up to 2^20
    ({"dtype": B.LCE_BF16, "D": 1 << 20}, B.LCE_OK),
    ({"dtype": B.LCE_BF16, "D": (1 << 20) + 8}, B.LCE_ERR_UNSUPPORTED),
    ({"N": 1 << 21, "chunk_rows": 1 << 20}, B.LCE_OK),
    ({"N": 1 << 21, "chunk_rows": (1 << 20) + 1}, B.LCE_ERR_UNSUPPORTED),
    ({"N": 1 << 21, "chunk_rows": B.LCE_CHUNK_ALL}, B.LCE_ERR_UNSUPPORTED),
    ({"V": (1 << 21) - 256}, B.LCE_OK),                 # fp32 W^T for grad_X
    ({"V": (1 << 21) - 255}, B.LCE_ERR_UNSUPPORTED),
    ({"V": (1 << 21) - 255, "flags": B.LCE_GRAD_W | B.LCE_GRAD_B}, B.LCE_OK),
    ({"V": 1 << 22, "dtype": B.LCE_BF16}, B.LCE_OK),    # 16-bit grad_X reads W in place
])
def test_create_validation(lib, kw, status):
    assert B.lce_create_status(_desc(**kw)) == status


@pytest.mark.parametrize("N,D,V,chunk", [
    # aspect_ratio rule of the LinearCrossEntropyOptions page (chunking_method):
    # next_pow2(ceil(N / ceil(V / D))), capped here at N rows.
    (256, 64, 1000, 16),          # ceil(1000/64)=16, 256/16=16
    (4096, 2048, 32000, 256),     # ceil(32000/2048)=16, 4096/16=256
    (8192, 4096, 128256, 256),    # ceil(128256/4096)=32, 8192/32=256
    (16384, 4096, 151936, 512),   # ceil(151936/4096)=38, ceil(16384/38)=432 -> 512
    (100, 64, 64, 100),           # ceil(64/64)=1 -> next_pow2(100)=128, capped at N
    (5, 8, 1000, 1),              # ceil(1000/8)=125, ceil(5/125)=1
])
def test_aspect_ratio_chunking(lib, N, D, V, chunk):
    h = B.lce_create(_desc(N=N, D=D, V=V, chunk_rows=B.LCE_CHUNK_ASPECT_RATIO,
                           dtype=B.LCE_BF16))
    try:
        c, n = B.lce_chunk_info(h)
        assert c == chunk and n == -(-N // chunk)
    finally:
        B.lce_destroy(h)


def test_explicit_and_single_chunk(lib):
    for rows, expect in ((64, (64, 4)), (3, (3, 86)), (1000, (256, 1)), (B.LCE_CHUNK_ALL, (256, 1))):
        h = B.lce_create(_desc(chunk_rows=rows))
        assert B.lce_chunk_info(h) == expect
        B.lce_destroy(h)
    h = B.lce_create(_desc(N=0))
    assert B.lce_chunk_info(h) == (0, 0)
    B.lce_destroy(h)


def test_workspace_grows_with_requested_outputs(lib):
    sizes = []
    for flags in (0, B.LCE_GRAD_B, B.LCE_GRAD_X | B.LCE_GRAD_B,
                  B.LCE_GRAD_X | B.LCE_GRAD_W | B.LCE_GRAD_B):
        h = B.lce_create(_desc(flags=flags))
        sizes.append(B.lce_workspace_size(h))
        B.lce_destroy(h)
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    # bf16 accurate keeps an fp32 V x D accumulator that compact does not
    acc = B.lce_create(_desc(dtype=B.LCE_BF16, acc_policy=B.LCE_ACCURATE))
    cmp_ = B.lce_create(_desc(dtype=B.LCE_BF16, acc_policy=B.LCE_COMPACT))
    assert B.lce_workspace_size(acc) - B.lce_workspace_size(cmp_) >= 1000 * 64 * 4
    # the non-mixed layout (bf16 accumulator) plans like compact, whatever the policy
    nm = B.lce_create(_desc(dtype=B.LCE_BF16, acc_dtype=B.LCE_BF16, acc_policy=B.LCE_ACCURATE))
    assert B.lce_workspace_size(nm) == B.lce_workspace_size(cmp_)
    B.lce_destroy(nm)
    B.lce_destroy(acc)
    B.lce_destroy(cmp_)


def test_forward_backward_host_validation(lib):
    """Errors found on the host return before anything is enqueued."""
    h = B.lce_create(_desc())
    ws = B.lce_workspace_size(h)
    fake = 1 << 20   # never dereferenced: validation fails first
    good = dict(X=fake, W=fake, b=fake, targets=fake, loss=fake, grad_X=fake, grad_W=fake,
                grad_b=fake, grad_scale=1.0)
    st = B.lce_forward_backward_status
    assert st(h, B.lce_io(**good), 0, ws, 0) == B.LCE_ERR_WORKSPACE
    assert st(h, B.lce_io(**good), fake, ws - 1, 0) == B.LCE_ERR_WORKSPACE
    assert st(h, B.lce_io(**good), fake + 16, ws, 0) == B.LCE_ERR_WORKSPACE
    assert st(h, B.lce_io(**{**good, "grad_W": None}), fake, ws, 0) == B.LCE_ERR_INVALID_ARG
    assert st(h, B.lce_io(**{**good, "b": None}), fake, ws, 0) == B.LCE_ERR_INVALID_ARG
    assert st(h, B.lce_io(**{**good, "loss": None}), fake, ws, 0) == B.LCE_ERR_INVALID_ARG
    assert st(h, B.lce_io(**{**good, "grad_output": fake}), fake, ws, 0) == B.LCE_ERR_INVALID_ARG
    assert st(h, B.lce_io(**{**good, "X": fake + 2}), fake, ws, 0) == B.LCE_ERR_UNSUPPORTED
    B.lce_destroy(h)


def test_status_strings_and_ce_workspace(lib):
    names = [B.lce_status_string(s) for s in range(6)]
    assert names == ["LCE_OK", "LCE_ERR_INVALID_ARG", "LCE_ERR_DTYPE", "LCE_ERR_UNSUPPORTED",
                     "LCE_ERR_WORKSPACE", "LCE_ERR_HIP"]
    assert B.lce_ce_workspace_size(16384, 131072) >= 3 * 16384 * 4
    with pytest.raises(lce.LceError):
        B.lce_ce_workspace_size(-1, 10)


def test_torch_wrapper_type_checks():
    """The pages' TypeError for non-int64 targets and RuntimeError for a bad
    bias shape, raised on the host before any device work."""
    import torch
    from linear_cross_entropy_chunk_amd.api import LinearCrossEntropy
    op = LinearCrossEntropy.__new__(LinearCrossEntropy)
    op.shape, op.dtype, op.bias, op.device = (4, 8, 10), torch.float32, True, torch.device("cpu")
    X, W = torch.zeros(4, 8), torch.zeros(10, 8)
    with pytest.raises(TypeError):
        op.check_inputs(X, W, torch.zeros(4, dtype=torch.int32), torch.zeros(10))
    with pytest.raises(RuntimeError):
        op.check_inputs(X, W, torch.zeros(4, dtype=torch.int64), torch.zeros(9))


def _ws(**kw) -> int:
    h = B.lce_create(_desc(**kw))
    try:
        return B.lce_workspace_size(h)
    finally:
        B.lce_destroy(h)


def test_group_rows_selects_the_per_chunk_path(lib):
    """group_rows caps the rows of dL held for one grad_W GEMM.  At the
    large-vocabulary shape (N=8192, D=4096, V=128256, bf16, 2048-row chunks):
    the default groups all four chunks (T holds all 8192 rows of dL, no fp32
    accumulator); group_rows=2048 holds one chunk of dL and an fp32 V x D
    accumulator; 4096 holds two chunks and the accumulator; compact ignores
    it.  Small regions (row statistics, staged X^T) stay below 0.2 GB."""
    N, D, V, c = 8192, 4096, 128256, 2048
    kw = dict(N=N, D=D, V=V, chunk_rows=c, dtype=B.LCE_BF16, has_bias=0,
              flags=B.LCE_GRAD_X | B.LCE_GRAD_W)
    slack = 0.2e9
    grouped = _ws(**kw)
    assert N * V * 2 <= grouped < N * V * 2 + slack
    assert _ws(group_rows=0, **kw) == grouped
    assert _ws(group_rows=N, **kw) == grouped
    acc = V * D * 4
    per_chunk = _ws(group_rows=c, **kw)
    assert c * V * 2 + acc <= per_chunk < c * V * 2 + acc + slack
    assert _ws(group_rows=1, **kw) == per_chunk          # below a chunk: one chunk
    assert _ws(group_rows=c + 100, **kw) == per_chunk    # rounded down to whole chunks
    two = _ws(group_rows=2 * c, **kw)
    assert 2 * c * V * 2 + acc <= two < 2 * c * V * 2 + acc + slack
    compact = _ws(acc_policy=B.LCE_COMPACT, **kw)
    assert _ws(acc_policy=B.LCE_COMPACT, group_rows=c, **kw) == compact
    assert compact < c * V * 2 + slack
    assert B.lce_create_status(_desc(group_rows=-1)) == B.LCE_ERR_INVALID_ARG


def test_torch_wrapper_device_shape_and_layout_checks():
    """Every tensor whose pointer reaches a kernel is checked on the host:
    device, shape, dtype and contiguity (a host or short target buffer
    would otherwise be read by the kernels).  'meta' tensors stand for the
    op's device here, where no GPU exists."""
    import torch
    from linear_cross_entropy_chunk_amd.api import CrossEntropyInplace, LinearCrossEntropy
    meta = torch.device("meta")
    op = LinearCrossEntropy.__new__(LinearCrossEntropy)
    op.shape, op.dtype, op.bias, op.device = (4, 8, 10), torch.float32, False, meta
    X, W = torch.empty(4, 8, device=meta), torch.empty(10, 8, device=meta)
    t = torch.empty(4, dtype=torch.int64, device=meta)
    op.check_inputs(X, W, t)                                   # all good: no error
    with pytest.raises(RuntimeError, match="target is on cpu"):
        op.check_inputs(X, W, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(RuntimeError, match="contiguous"):
        op.check_inputs(X, W, torch.empty(8, dtype=torch.int64, device=meta)[::2])
    with pytest.raises(RuntimeError):
        op.check_inputs(X, W, torch.empty(3, dtype=torch.int64, device=meta))
    with pytest.raises(RuntimeError, match="X is on cpu"):
        op.check_inputs(torch.zeros(4, 8), W, t)
    with pytest.raises(RuntimeError, match="contiguous"):
        op.check_inputs(torch.empty(8, 4, device=meta).t(), W, t)
    with pytest.raises(RuntimeError, match="grad_output is on cpu"):
        op.check_inputs(X, W, t, grad_output=torch.zeros(4))
    with pytest.raises(RuntimeError, match="grad_output must have shape"):
        op.check_inputs(X, W, t, grad_output=torch.empty(5, device=meta))
    with pytest.raises(RuntimeError, match="contiguous"):
        op.check_inputs(X, W, t, grad_output=torch.empty(8, device=meta)[::2])
    with pytest.raises(RuntimeError, match="grad_output must be torch.float32"):
        op.check_inputs(X, W, t, grad_output=torch.empty(4, dtype=torch.float16, device=meta))

    ce = CrossEntropyInplace.__new__(CrossEntropyInplace)
    ce.N, ce.V, ce.device, ce.reduction, ce.ignore_index = 4, 16, meta, "mean", -100
    z = torch.empty(4, 16, device=meta)
    with pytest.raises(RuntimeError, match="target is on cpu"):
        ce(z, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(RuntimeError, match="logits is on cpu"):
        ce(torch.zeros(4, 16), t)
    with pytest.raises(RuntimeError, match="target must have shape"):
        ce(z, torch.empty(3, dtype=torch.int64, device=meta))
    with pytest.raises(RuntimeError, match="contiguous"):
        ce(z, torch.empty(8, dtype=torch.int64, device=meta)[::2])
    with pytest.raises(RuntimeError, match="logits must have shape"):
        ce(torch.empty(4, 12, device=meta), t)
