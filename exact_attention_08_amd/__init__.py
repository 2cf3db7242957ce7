"""MI355X-native exact attention: gfx950 HIP kernels behind a C ABI
(include/fa.h, libfa355.so) and this thin binding.

Forward: ``fwd`` (padded batch, causal / sliding window / GQA), ``fwd_mod``
(ALiBi bias, soft-capping), ``fwd_varlen`` (packed sequences), ``fwd_fp8``
(8-bit e4m3 inputs).  Decode: ``decode_kvcache`` (contiguous cache, split
keys), ``decode_kvcache_noalloc`` (the same with the library's own scratch
array, for callers that cannot allocate), ``decode_paged`` (paged cache with
in-place append).  Gradients: ``bwd``.  The ``*_workspace_bytes`` helpers give
the caller-provided workspace sizes.

Importing the package does not load the library; the first call does and
raises if it is not built: there is no fallback.  ``using(path)`` runs calls
on another build of the library (the checking build ``DEBUG_LIB_PATH``).
"""
from .fa import (DEBUG_LIB_PATH, DECODE_NOALLOC_MAX_BYTES, LIB_PATH, FAError,  # noqa: F401
                 bwd, bwd_workspace_bytes, decode_kvcache, decode_kvcache_noalloc, decode_paged,
                 decode_workspace_bytes, fwd, fwd_fp8, fwd_fp8_workspace_bytes, fwd_mod,
                 fwd_varlen, load, using)

__all__ = ["fwd", "fwd_mod", "fwd_varlen", "fwd_fp8", "fwd_fp8_workspace_bytes",
           "decode_kvcache", "decode_kvcache_noalloc", "decode_paged", "decode_workspace_bytes",
           "bwd", "bwd_workspace_bytes", "load", "using", "FAError", "LIB_PATH", "DEBUG_LIB_PATH",
           "DECODE_NOALLOC_MAX_BYTES"]
