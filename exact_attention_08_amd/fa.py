"""Python binding of libfa355.so (include/fa.h) over torch tensors.

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, the current torch stream, and a ctypes call into the C ABI.  Every
step of the attention itself runs in the library's HIP kernels.  There is no
fallback: if the library is missing or a call fails, a RuntimeError says so.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa355.so")
# The checking build of the same sources (every copy-pipeline wait drained,
# LDS rings filled with NaN before first use): for tests that compare it with
# the pipelined library bit for bit.
DEBUG_LIB_PATH = os.path.join(_PKG, "libfa355_debug.so")

FA_BF16, FA_FP16 = 0, 1
_DTYPE = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16}
STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED", 3: "FA_ERR_WORKSPACE",
          4: "FA_ERR_HIP"}

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_mod", "fa_fwd_fp8_workspace_bytes", "fa_fwd_fp8", "fa_fwd_varlen", "fa_decode_workspace_bytes", "fa_decode_kvcache",
           "fa_decode_kvcache_noalloc", "fa_decode_paged", "fa_bwd_workspace_bytes", "fa_bwd", "fa_status_str",
           "fa_last_error")

_lock = threading.Lock()
_libs: dict = {}
_active = threading.local()     # path of the library calls go to (default LIB_PATH)


class FAError(RuntimeError):
    """A non-OK status returned by the C ABI."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load a built library (default: the one calls currently go to) and
    declare its C signatures."""
    if path is None:
        path = getattr(_active, "path", None) or LIB_PATH
    with _lock:
        if path in _libs:
            return _libs[path]
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: the HIP library is not built "
                "(run __graft_entry__.build()); there is no fallback path")
        lib = ctypes.CDLL(path)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P]
        lib.fa_fwd.restype = I
        lib.fa_fwd_mod.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P, F, I, P]
        lib.fa_fwd_mod.restype = I
        lib.fa_fwd_fp8_workspace_bytes.argtypes = [I, I, I, I]
        lib.fa_fwd_fp8_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, F, F, F, P,
                                   ctypes.c_size_t, P]
        lib.fa_fwd_fp8.restype = I
        lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, I, P]
        lib.fa_fwd_varlen.restype = I
        lib.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_decode_kvcache.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P,
                                          ctypes.c_size_t, I, P]
        lib.fa_decode_kvcache.restype = I
        lib.fa_decode_kvcache_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F,
                                                  I, I, P]
        lib.fa_decode_kvcache_noalloc.restype = I
        lib.fa_decode_paged.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I,
                                        F, I, P, ctypes.c_size_t, I, P]
        lib.fa_decode_paged.restype = I
        lib.fa_bwd_workspace_bytes.argtypes = [I, I, I]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P,
                               ctypes.c_size_t, I, P]
        lib.fa_bwd.restype = I
        lib.fa_status_str.argtypes = [I]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_last_error.argtypes = []
        lib.fa_last_error.restype = ctypes.c_char_p
        _libs[path] = lib
        return lib


@contextlib.contextmanager
def using(path: str):
    """Route this thread's calls to the library at path (e.g. DEBUG_LIB_PATH)
    inside the block."""
    old = getattr(_active, "path", None)
    _active.path = path
    try:
        yield load(path)
    finally:
        _active.path = old


def _check(status: int) -> None:
    if status != 0:
        raise FAError(status, load().fa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _scale(softmax_scale, d: int) -> float:
    # None -> 1/sqrt(head_dim), as flash_attn_func's softmax_scale=None
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensors(*ts):
    dt = ts[0].dtype
    _require(dt in _DTYPE, f"dtype {dt} unsupported (bf16 or fp16)")
    for t in ts:
        _require(t.is_cuda, "tensors must be on a GPU")
        _require(t.dtype == dt, "q, k, v must share one dtype")
        _require(t.is_contiguous(), "tensors must be contiguous")


def fwd(q, k, v, *, causal=False, window=(-1, -1), softmax_scale=None, out=None, lse=None):
    """Padded batch: q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] -> (out [B,Sq,Hq,d], lse [B,Hq,Sq] fp32)."""
    _check_tensors(q, k, v)
    _require(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "expected 4-d q, k, v")
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    _require(k.shape[0] == B and k.shape[3] == d, "k/v batch or head_dim mismatch")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check(load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                         int(bool(causal)), int(window[0]), int(window[1]),
                         _scale(softmax_scale, d), _DTYPE[q.dtype], _stream()))
    return out, lse


def fwd_mod(q, k, v, *, causal=False, window=(-1, -1), softmax_scale=None, alibi_slopes=None,
            softcap=0.0, out=None, lse=None):
    """fwd() with score modifiers: alibi_slopes (fp32 [Hq] GPU tensor, bias
    -slope_h * |pos_i - j|) and softcap (cap * tanh(s / cap), 0 = off)."""
    _check_tensors(q, k, v)
    _require(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "expected [B,S,H,d] q, k, v")
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    if alibi_slopes is not None:
        _require(alibi_slopes.is_cuda and alibi_slopes.dtype == torch.float32
                 and alibi_slopes.is_contiguous() and alibi_slopes.numel() == Hq,
                 "alibi_slopes must be a contiguous fp32 [Hq] GPU tensor")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    lib = load()
    _check(lib.fa_fwd_mod(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                          int(bool(causal)), int(window[0]), int(window[1]),
                          _scale(softmax_scale, d), _ptr(alibi_slopes), float(softcap),
                          _DTYPE[q.dtype], _stream()))
    return out, lse


def fwd_fp8_workspace_bytes(B: int, Hkv: int, Sk: int, d: int) -> int:
    return int(load().fa_fwd_fp8_workspace_bytes(B, Hkv, Sk, d))


def fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, *, causal=False, window=(-1, -1),
            softmax_scale=None, out=None, lse=None, workspace=None):
    """8-bit forward: q8 [B,Sq,Hq,d], k8/v8 [B,Sk,Hkv,d] uint8 e4m3 codes on the GPU with
    per-tensor descales -> (out [B,Sq,Hq,d] bf16, lse [B,Hq,Sq] fp32)."""
    for t in (q8, k8, v8):
        _require(t.is_cuda and t.dtype == torch.uint8 and t.is_contiguous() and t.dim() == 4,
                 "q8, k8, v8 must be contiguous 4-d uint8 GPU tensors (e4m3 codes)")
    _require(k8.shape == v8.shape, "k8 and v8 must have one shape")
    B, Sq, Hq, d = q8.shape
    _, Sk, Hkv, _ = k8.shape
    lib = load()
    need = int(lib.fa_fwd_fp8_workspace_bytes(B, Hkv, Sk, d))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q8.device)
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    _check(lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk,
                          d, int(bool(causal)), int(window[0]), int(window[1]),
                          _scale(softmax_scale, d), float(descale_q), float(descale_k),
                          float(descale_v), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream()))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, causal=False,
               window=(-1, -1), softmax_scale=None, out=None, lse=None):
    """Packed: q [total_q,Hq,d], k/v [total_k,Hkv,d], cu_seqlens int32 [B+1] on the GPU
    -> (out [total_q,Hq,d], lse [Hq,total_q] fp32)."""
    _check_tensors(q, k, v)
    _require(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape, "expected 3-d q, k, v")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        _require(cu.is_cuda and cu.dtype == torch.int32 and cu.dim() == 1 and cu.is_contiguous(),
                 "cu_seqlens must be contiguous int32 GPU vectors")
    total_q, Hq, d = q.shape
    _, Hkv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    _require(B >= 1 and cu_seqlens_k.numel() == B + 1, "cu_seqlens must have B+1 entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check(load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv,
                                int(max_seqlen_q), int(max_seqlen_k), total_q, d,
                                int(bool(causal)), int(window[0]), int(window[1]),
                                _scale(softmax_scale, d), _DTYPE[q.dtype], _stream()))
    return out, lse


def decode_workspace_bytes(B: int, Hq: int, max_seqlen_k: int, d: int, split_size: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, Hq, max_seqlen_k, d, split_size))


def decode_kvcache(q, k_cache, v_cache, cache_seqlens, max_seqlen_k, *, causal=False,
                   window=(-1, -1), softmax_scale=None, split_size=1024, out=None, lse=None,
                   workspace=None):
    """One-token decode: q [B,1,Hq,d], caches [B,Sk_cap,Hkv,d], cache_seqlens int32 [B]
    on the GPU -> (out [B,1,Hq,d], lse [B,Hq] fp32).  The fp32 workspace is allocated
    with torch unless given (uint8 tensor of at least decode_workspace_bytes)."""
    _check_tensors(q, k_cache, v_cache)
    _require(q.dim() == 4 and q.shape[1] == 1, "q must be [B,1,Hq,d]")
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "caches must be [B,Sk_cap,Hkv,d]")
    _require(cache_seqlens.is_cuda and cache_seqlens.dtype == torch.int32,
             "cache_seqlens must be an int32 GPU vector")
    B, _, Hq, d = q.shape
    _, Sk_cap, Hkv, _ = k_cache.shape
    lib = load()
    need = int(lib.fa_decode_workspace_bytes(B, Hq, int(max_seqlen_k), d, int(split_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.fa_decode_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                 _ptr(out), _ptr(lse), B, Hq, Hkv, Sk_cap, int(max_seqlen_k), d,
                                 int(bool(causal)), int(window[0]), int(window[1]),
                                 _scale(softmax_scale, d), int(split_size), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _DTYPE[q.dtype], _stream()))
    return out, lse


# Largest partial-result size of decode_kvcache_noalloc (FA_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 64 << 20


def decode_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, max_seqlen_k, *, out, lse=None,
                           causal=False, window=(-1, -1), softmax_scale=None, split_size=1024):
    """decode_kvcache without a workspace: the library keeps the split partials in its
    own per-GPU scratch array (for callers that cannot allocate).  The caller passes
    out (and lse, or None); this function allocates nothing."""
    _check_tensors(q, k_cache, v_cache, out)
    _require(q.dim() == 4 and q.shape[1] == 1, "q must be [B,1,Hq,d]")
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "caches must be [B,Sk_cap,Hkv,d]")
    _require(out.shape == q.shape, "out must be shaped like q")
    _require(cache_seqlens.is_cuda and cache_seqlens.dtype == torch.int32,
             "cache_seqlens must be an int32 GPU vector")
    B, _, Hq, d = q.shape
    _, Sk_cap, Hkv, _ = k_cache.shape
    if lse is not None:
        _require(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
                 and tuple(lse.shape) == (B, Hq), "lse must be a contiguous fp32 [B,Hq] GPU tensor")
    _check(load().fa_decode_kvcache_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Hq,
        Hkv, Sk_cap, int(max_seqlen_k), d, int(bool(causal)), int(window[0]), int(window[1]),
        _scale(softmax_scale, d), int(split_size), _DTYPE[q.dtype], _stream()))
    return out, lse


def decode_paged(q, k_pages, v_pages, block_table, cache_seqlens, max_seqlen_k, *, k_new=None,
                 v_new=None, causal=False, window=(-1, -1), softmax_scale=None, split_size=1024,
                 out=None, lse=None, workspace=None):
    """One-token decode against a paged cache: q [B,1,Hq,d], page pools
    [num_pages,page_size,Hkv,d], block_table int32 [B,max_pages], cache_seqlens int32 [B]
    (tokens in the cache), optional k_new/v_new [B,1,Hkv,d] appended in place at
    position cache_seqlens[b] before attending -> (out [B,1,Hq,d], lse [B,Hq] fp32)."""
    _check_tensors(q, k_pages, v_pages)
    _require(q.dim() == 4 and q.shape[1] == 1, "q must be [B,1,Hq,d]")
    _require(k_pages.dim() == 4 and k_pages.shape == v_pages.shape,
             "page pools must be [num_pages,page_size,Hkv,d]")
    _require(block_table.is_cuda and block_table.dtype == torch.int32 and block_table.dim() == 2
             and block_table.is_contiguous(), "block_table must be a contiguous int32 [B,max_pages] GPU tensor")
    _require(cache_seqlens.is_cuda and cache_seqlens.dtype == torch.int32,
             "cache_seqlens must be an int32 GPU vector")
    B, _, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_pages.shape
    _require(block_table.shape[0] == B, "block_table must have B rows")
    if k_new is not None or v_new is not None:
        _require(k_new is not None and v_new is not None, "give both k_new and v_new")
        _check_tensors(k_new, v_new)
        _require(tuple(k_new.shape) == (B, 1, Hkv, d) and v_new.shape == k_new.shape,
                 "k_new, v_new must be [B,1,Hkv,d]")
    lib = load()
    need = int(lib.fa_decode_workspace_bytes(B, Hq, int(max_seqlen_k), d, int(split_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                               _ptr(cache_seqlens), _ptr(k_new) if k_new is not None else None,
                               _ptr(v_new) if v_new is not None else None, _ptr(out), _ptr(lse),
                               B, Hq, Hkv, num_pages, page_size, block_table.shape[1],
                               int(max_seqlen_k), d, int(bool(causal)), int(window[0]),
                               int(window[1]), _scale(softmax_scale, d), int(split_size),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _DTYPE[q.dtype], _stream()))
    return out, lse


def bwd_workspace_bytes(B: int, Hq: int, Sq: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, Hq, Sq))


def bwd(q, k, v, out, dout, lse, *, causal=False, window=(-1, -1), softmax_scale=None,
        dq=None, dk=None, dv=None, workspace=None):
    """Gradients of the padded-batch attention: q, out, dout [B,Sq,Hq,d], k/v [B,Sk,Hkv,d],
    lse [B,Hq,Sq] fp32 from fwd() -> (dq, dk, dv).  The fp32 workspace is allocated with
    torch unless given (uint8 tensor of at least bwd_workspace_bytes)."""
    _check_tensors(q, k, v, out, dout)
    _require(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "expected 4-d q, k, v")
    _require(out.shape == q.shape and dout.shape == q.shape, "out and dout must match q")
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    _require(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
             and tuple(lse.shape) == (B, Hq, Sq), "lse must be a contiguous fp32 [B,Hq,Sq] GPU tensor")
    lib = load()
    need = int(lib.fa_bwd_workspace_bytes(B, Hq, Sq))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                      _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Sk, d, int(bool(causal)),
                      int(window[0]), int(window[1]), _scale(softmax_scale, d), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _DTYPE[q.dtype], _stream()))
    return dq, dk, dv
