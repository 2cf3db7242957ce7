"""MI355X-native fused exact-attention forward (gfx950 HIP kernels behind a C ABI).

``fwd``, ``fwd_varlen`` and ``decode_kvcache`` call ``libfa355.so``; importing
the package does not load the library, the first call does (and raises if it
is not built: there is no fallback).
"""
from .fa import (FAError, decode_kvcache, decode_workspace_bytes, fwd,  # noqa: F401
                 fwd_varlen, load)

__all__ = ["fwd", "fwd_varlen", "decode_kvcache", "decode_workspace_bytes", "load", "FAError"]
