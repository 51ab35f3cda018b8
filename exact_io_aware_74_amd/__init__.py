"""Exact scaled-dot-product attention for MI355X (gfx950).

The computation lives in libfa.so (hand-written HIP kernels behind the C ABI
of include/fa.h); this package is its thin Python binding. Importing the
package does not load the library; the first call does, and raises if the
library has not been built.
"""
from .binding import (FaError, decode, decode_workspace_bytes, default_scale, fwd, load, naive_fwd,
                      naive_workspace_bytes, shutdown)

__all__ = ["fwd", "decode", "naive_fwd", "naive_workspace_bytes", "decode_workspace_bytes", "default_scale",
           "shutdown", "load", "FaError"]
