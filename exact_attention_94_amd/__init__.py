"""Exact attention (FlashAttention-style forward and recompute backward) for AMD MI355X.

The computation lives in libfa.so (hand-written HIP kernels for gfx950, C ABI in include/fa.h);
this package only builds and binds it.
"""

from .binding import (FA_BF16, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_RANGE, FA_ERR_UNSUPPORTED,
                      FA_ERR_WORKSPACE, FA_F16, FA_F32, FA_OK, FAError, backward, decode,
                      decode_workspace_bytes, forward, status_string, workspace_bytes)

__all__ = ["forward", "backward", "decode", "workspace_bytes", "decode_workspace_bytes",
           "status_string", "FAError", "FA_OK",
           "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
           "FA_ERR_RANGE", "FA_F32",
           "FA_F16", "FA_BF16"]
