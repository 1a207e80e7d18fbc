"""Host-side behaviour of the autograd entry points and of lce_scale (no GPU,
no compute call): the options of the LinearCrossEntropyOptions page resolved
into the C descriptor, the chunk rows the library plans for "aspect_ratio"
and "aspect_ratio:N" against their closed form, and the argument errors the
pages' Python raises."""
import math

import pytest
import torch

from linear_cross_entropy_chunk_amd import LinearCrossEntropyOptions, LceError
from linear_cross_entropy_chunk_amd import _binding as B
from linear_cross_entropy_chunk_amd.functional import _resolve, linear_cross_entropy


def _planned_rows(N, D, V, chunk_rows, divisor=1):
    d = B.lce_desc(N=N, D=D, V=V, ignore_index=-100, chunk_rows=chunk_rows, dtype=B.LCE_F32,
                   acc_dtype=B.LCE_F32, has_bias=0, reduction=B.LCE_MEAN,
                   acc_policy=B.LCE_ACCURATE, flags=B.LCE_GRAD_X, chunk_divisor=divisor)
    h = B.lce_create(d)
    try:
        return B.lce_chunk_info(h)[0]
    finally:
        B.lce_destroy(h)


def _next_pow2(x):
    return 1 << max(0, math.ceil(math.log2(x)))


@pytest.mark.parametrize("N,D,V", [(300, 64, 777), (8192, 4096, 128256), (16384, 4096, 151936),
                                   (5, 8, 3), (1000, 16, 100000)])
@pytest.mark.parametrize("divisor", [1, 2, 3, 4, 1000])
def test_aspect_ratio_rows_follow_the_closed_form(N, D, V, divisor):
    """next_pow2(ceil(N / ceil(V / D))), divided by N (floor, at least one
    row), never more than N."""
    base = _next_pow2(math.ceil(N / math.ceil(V / D)))
    want = min(N, max(1, base // divisor))
    assert _planned_rows(N, D, V, B.LCE_CHUNK_ASPECT_RATIO, divisor) == want


def test_negative_divisor_is_rejected():
    with pytest.raises(LceError):
        _planned_rows(10, 8, 8, B.LCE_CHUNK_ASPECT_RATIO, -1)


def test_options_resolution():
    N, D, V = 300, 64, 777
    f32 = torch.float32
    r = _resolve(LinearCrossEntropyOptions(), N, D, V, f32)
    assert r == {"chunk_rows": B.LCE_CHUNK_ASPECT_RATIO, "chunk_divisor": 1,
                 "acc_policy": "compact", "acc_dtype": torch.float32}
    r = _resolve(LinearCrossEntropyOptions(chunking_method="aspect_ratio:4",
                                           acc_policy="accurate"), N, D, V, f32)
    assert r["chunk_divisor"] == 4 and r["acc_policy"] == "accurate"
    # the default method yields to an explicit size; None uses the size or one chunk
    assert _resolve(LinearCrossEntropyOptions(batch_chunk_size=50), N, D, V, f32)[
        "chunk_rows"] == 50
    assert _resolve(LinearCrossEntropyOptions(chunking_method=None), N, D, V, f32)[
        "chunk_rows"] == B.LCE_CHUNK_ALL
    # an explicit method and a size that agree are accepted, disagreeing ones raise
    _resolve(LinearCrossEntropyOptions(chunking_method="aspect_ratio", batch_chunk_size=32),
             N, D, V, f32)
    with pytest.raises(ValueError):
        _resolve(LinearCrossEntropyOptions(chunking_method="aspect_ratio", batch_chunk_size=50),
                 N, D, V, f32)
    with pytest.raises(ValueError):
        _resolve(LinearCrossEntropyOptions(chunking_method="balanced"), N, D, V, f32)
    with pytest.raises(ValueError):
        _resolve(LinearCrossEntropyOptions(acc_policy="fast"), N, D, V, f32)
    # acc_dtype: float32 (mixed precision), or the input dtype itself (the
    # non-mixed layout, which accumulates like "compact" whatever the policy);
    # any other dtype is an error
    with pytest.raises(RuntimeError):
        _resolve(LinearCrossEntropyOptions(acc_dtype=torch.bfloat16), N, D, V, f32)
    with pytest.raises(RuntimeError):
        _resolve(LinearCrossEntropyOptions(acc_dtype=torch.float16), N, D, V, torch.bfloat16)
    for dt in (torch.bfloat16, torch.float16):
        r = _resolve(LinearCrossEntropyOptions(acc_dtype=dt, acc_policy="accurate"), N, D, V, dt)
        assert r["acc_dtype"] == dt and r["acc_policy"] == "compact"
    r = _resolve(LinearCrossEntropyOptions(acc_dtype=torch.float32, acc_policy="accurate"),
                 N, D, V, torch.float16)
    assert r["acc_dtype"] == torch.float32 and r["acc_policy"] == "accurate"
    assert _resolve(LinearCrossEntropyOptions(acc_dtype=f32), N, D, V, f32)["acc_dtype"] == f32


def test_argument_errors_before_any_device_work():
    X = torch.zeros(4, 8)
    W = torch.zeros(6, 8)
    t = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(TypeError):
        linear_cross_entropy(X, W, t.to(torch.int32))
    with pytest.raises(RuntimeError):
        linear_cross_entropy(X, W, t, torch.zeros(5))
    with pytest.raises(NotImplementedError):
        linear_cross_entropy(X, W, t, label_smoothing=0.1)
    with pytest.raises(NotImplementedError):             # [LCE]: unsupported reduction
        linear_cross_entropy(X, W, t, reduction="max")
    with pytest.raises(NotImplementedError):
        linear_cross_entropy(X.double(), W.double(), t)
    with pytest.raises(RuntimeError):
        linear_cross_entropy(X, W, torch.zeros(5, dtype=torch.int64))


def test_scale_validates_on_the_host():
    stream = 0
    with pytest.raises(LceError):                       # unknown dtype
        B.lce_scale(256, 256, 7, 1, 8, 256, 0, stream)
    with pytest.raises(LceError):                       # negative size
        B.lce_scale(256, 256, B.LCE_F32, -1, 8, 256, 0, stream)
    with pytest.raises(LceError):                       # misaligned
        B.lce_scale(260, 260, B.LCE_F32, 1, 8, 256, 0, stream)
    with pytest.raises(LceError):                       # rows of 6 bf16 with per-row scale
        B.lce_scale(256, 256, B.LCE_BF16, 2, 6, 256, 1, stream)
    B.lce_scale(0, 0, B.LCE_F32, 0, 8, 0, 0, stream)    # nothing to do: no device call
