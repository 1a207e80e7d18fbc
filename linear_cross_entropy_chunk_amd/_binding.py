"""ctypes binding of liblce.so: the C ABI of include/lce.h, same names,
argument marshalling only.  Every step of the computation runs in the HIP
library; if the library is missing or fails to load, every call raises."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblce.so")

# enums of lce.h
LCE_OK, LCE_ERR_INVALID_ARG, LCE_ERR_DTYPE, LCE_ERR_UNSUPPORTED, LCE_ERR_WORKSPACE, LCE_ERR_HIP = range(6)
LCE_F32, LCE_BF16, LCE_F16 = 0, 1, 2
LCE_MEAN, LCE_SUM, LCE_NONE = 0, 1, 2
LCE_ACCURATE, LCE_COMPACT = 0, 1
LCE_GRAD_X, LCE_GRAD_W, LCE_GRAD_B, LCE_ARGMAX, LCE_ACCUMULATE = 1, 2, 4, 8, 16
LCE_CHUNK_ASPECT_RATIO, LCE_CHUNK_ALL = 0, -1

# Every exported function of include/lce.h.
EXPORTS = ("lce_create", "lce_workspace_size", "lce_chunk_info", "lce_forward_backward",
           "lce_destroy", "lce_ce_workspace_size", "lce_ce_inplace", "lce_timing_enable",
           "lce_timing_read", "lce_status_string", "lce_last_error", "lce_scale",
           "lce_ce_inplace_noalloc")
LCE_CE_NOALLOC_MAX_ROWS = 1 << 20

# kernel classes of the timing hook
KERNEL_CLASSES = ("prep", "logits", "combine", "finalize", "gemm_x", "split_sum", "transpose",
                  "gemm_w", "bias", "loss", "repair")
LCE_K_COUNT = len(KERNEL_CLASSES)


class lce_desc(ctypes.Structure):
    _fields_ = [("N", c_int64), ("D", c_int64), ("V", c_int64), ("ignore_index", c_int64),
                ("chunk_rows", c_int64), ("dtype", c_int32), ("acc_dtype", c_int32),
                ("has_bias", c_int32), ("reduction", c_int32), ("acc_policy", c_int32),
                ("flags", c_uint32), ("chunk_divisor", c_int64), ("group_rows", c_int64)]


class lce_io(ctypes.Structure):
    _fields_ = [("X", c_void_p), ("W", c_void_p), ("b", c_void_p), ("targets", c_void_p),
                ("grad_output", c_void_p), ("loss", c_void_p), ("grad_X", c_void_p),
                ("grad_W", c_void_p), ("grad_b", c_void_p), ("argmax", c_void_p),
                ("n_valid", c_void_p), ("n_bad", c_void_p), ("grad_scale", c_float),
                ("reserved", c_int32), ("class_weight", c_void_p)]


class LceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {lce_status_string(status)}"
        detail = lce_last_error()
        if status == LCE_ERR_HIP or (detail and detail.startswith(where)):
            msg += f" ({detail})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if liblce.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_cross_entropy_chunk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.lce_create.argtypes = [POINTER(lce_desc), POINTER(c_void_p)]
        L.lce_workspace_size.argtypes = [c_void_p, POINTER(c_size_t)]
        L.lce_chunk_info.argtypes = [c_void_p, POINTER(c_int64), POINTER(c_int64)]
        L.lce_forward_backward.argtypes = [c_void_p, POINTER(lce_io), c_void_p, c_size_t, c_void_p]
        L.lce_destroy.argtypes = [c_void_p]
        L.lce_ce_workspace_size.argtypes = [c_int64, c_int64, POINTER(c_size_t)]
        L.lce_ce_inplace.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                     c_int32, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                     c_void_p]
        L.lce_scale.argtypes = [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_void_p, c_int64,
                                c_void_p]
        L.lce_ce_inplace_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                             c_int64, c_int32, c_float, c_void_p, c_void_p,
                                             c_void_p]
        L.lce_timing_enable.argtypes = [c_void_p, c_uint32]
        L.lce_timing_read.argtypes = [c_void_p, POINTER(ctypes.c_double), POINTER(c_int64)]
        L.lce_status_string.argtypes = [c_int32]
        L.lce_status_string.restype = c_char_p
        L.lce_last_error.argtypes = []
        L.lce_last_error.restype = c_char_p
        for name in EXPORTS:
            if name not in ("lce_status_string", "lce_last_error"):
                getattr(L, name).restype = c_int32
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != LCE_OK:
        raise LceError(status, where)


def lce_status_string(status: int) -> str:
    return lib().lce_status_string(status).decode()


def lce_last_error() -> str:
    return lib().lce_last_error().decode()


def lce_create(desc: lce_desc) -> c_void_p:
    h = c_void_p()
    _check(lib().lce_create(byref(desc), byref(h)), "lce_create")
    return h


def lce_create_status(desc: lce_desc) -> int:
    """lce_create returning the raw status (for validation tests)."""
    h = c_void_p()
    st = lib().lce_create(byref(desc), byref(h))
    if st == LCE_OK:
        lib().lce_destroy(h)
    return st


def lce_workspace_size(handle) -> int:
    n = c_size_t()
    _check(lib().lce_workspace_size(handle, byref(n)), "lce_workspace_size")
    return n.value


def lce_chunk_info(handle) -> tuple[int, int]:
    c, k = c_int64(), c_int64()
    _check(lib().lce_chunk_info(handle, byref(c), byref(k)), "lce_chunk_info")
    return c.value, k.value


def lce_forward_backward(handle, io: lce_io, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().lce_forward_backward(handle, byref(io), c_void_p(workspace), ws_bytes,
                                      c_void_p(stream)), "lce_forward_backward")


def lce_forward_backward_status(handle, io: lce_io, workspace: int, ws_bytes: int,
                                stream: int) -> int:
    return lib().lce_forward_backward(handle, byref(io), c_void_p(workspace), ws_bytes,
                                      c_void_p(stream))


def lce_destroy(handle) -> None:
    _check(lib().lce_destroy(handle), "lce_destroy")


def lce_ce_workspace_size(N: int, V: int) -> int:
    n = c_size_t()
    _check(lib().lce_ce_workspace_size(N, V, byref(n)), "lce_ce_workspace_size")
    return n.value


def lce_ce_inplace(logits: int, targets: int, class_weight: int | None, N: int, V: int,
                   ignore_index: int, reduction: int, grad_scale: float, loss: int,
                   n_valid: int, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().lce_ce_inplace(c_void_p(logits), c_void_p(targets),
                                c_void_p(class_weight or None), N, V, ignore_index,
                                reduction, grad_scale, c_void_p(loss), c_void_p(n_valid or None),
                                c_void_p(workspace), ws_bytes, c_void_p(stream)),
           "lce_ce_inplace")


def lce_ce_inplace_noalloc(logits: int, targets: int, class_weight: int | None, N: int, V: int,
                           ignore_index: int, reduction: int, grad_scale: float, loss: int,
                           n_valid: int, stream: int) -> None:
    _check(lib().lce_ce_inplace_noalloc(c_void_p(logits), c_void_p(targets),
                                        c_void_p(class_weight or None), N, V, ignore_index,
                                        reduction, grad_scale, c_void_p(loss),
                                        c_void_p(n_valid or None), c_void_p(stream)),
           "lce_ce_inplace_noalloc")


def lce_ce_inplace_noalloc_status(logits: int, targets: int, N: int, V: int, reduction: int,
                                  loss: int) -> int:
    """lce_ce_inplace_noalloc returning the raw status (host validation tests)."""
    return lib().lce_ce_inplace_noalloc(c_void_p(logits), c_void_p(targets), None, N, V, -100,
                                        reduction, 1.0, c_void_p(loss), None, None)


def lce_scale(src: int, dst: int, dtype: int, rows: int, cols: int, scale: int,
              scale_stride: int, stream: int) -> None:
    _check(lib().lce_scale(c_void_p(src or None), c_void_p(dst or None), dtype, rows, cols,
                           c_void_p(scale or None), scale_stride, c_void_p(stream)),
           "lce_scale")


def lce_timing_enable(handle, kernel_mask: int) -> None:
    _check(lib().lce_timing_enable(handle, kernel_mask), "lce_timing_enable")


def lce_timing_read(handle) -> dict:
    """{class name: (total ms, launches)} since the last read."""
    ms = (ctypes.c_double * LCE_K_COUNT)()
    n = (c_int64 * LCE_K_COUNT)()
    _check(lib().lce_timing_read(handle, ms, n), "lce_timing_read")
    return {KERNEL_CLASSES[k]: (ms[k], n[k]) for k in range(LCE_K_COUNT)}
