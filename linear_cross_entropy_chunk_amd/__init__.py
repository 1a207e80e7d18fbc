"""Chunked fused linear-cross-entropy for AMD MI355X (gfx950).

The computation lives in liblce.so (hand-written HIP kernels behind the C ABI
of include/lce.h); this package is its Python binding.  There is no CPU or
PyTorch fallback: without the built library every call raises.
"""
from ._binding import (EXPORTS, LIB_PATH, LceError, lce_ce_inplace,  # noqa: F401
                       lce_ce_workspace_size, lce_chunk_info, lce_create, lce_destroy,
                       lce_forward_backward, lce_last_error, lce_status_string,
                       lce_workspace_size)
from .api import (CrossEntropyInplace, LinearCrossEntropy,  # noqa: F401
                  cross_entropy_inplace, linear_cross_entropy)
from .functional import LinearCrossEntropyOptions  # noqa: F401
from . import functional  # noqa: F401
