"""fp64 CPU attention oracle: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this module.  The GPU library never imports, links or calls it, and
this module imports nothing from the GPU package.

The arithmetic lives in ``fa_oracle.c`` (plain double-precision definition of
attention; see the header of that file for the passages it follows and the
readings taken where the pages are silent).  This module only builds that
file with gcc, converts inputs exactly to float64 and marshals arguments.

Every input is converted with an exact widening cast (bf16/fp16/fp32 to
fp64), so the oracle sees precisely the values the GPU sees.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "fa_oracle.c")
LIB = os.path.join(_HERE, "libfa_oracle.so")

_lock = threading.Lock()
_lib_cache: dict[str, ctypes.CDLL] = {}


def build(src: str = SRC, out: str = LIB, extra_flags: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over rows)."""
    # build beside the target, then rename: a process loading the library
    # meanwhile sees either the old file or the new one, never a partial one
    tmp = f"{out}.{os.getpid()}.tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.fa_oracle_rows.argtypes = [P, i64, P, i32, i64, P, P, i64, i64, i32,
                                   i32, i32, i32, f64, P, i64, P]
    lib.fa_oracle_fwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                  i32, i32, i32, f64]
    lib.fa_oracle_varlen.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32,
                                     i32, i32, i32, f64]
    lib.fa_oracle_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                     i32, i32, i32, f64]
    lib.fa_oracle_bwd.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                  i32, i32, i32, f64]
    lib.fa_oracle_decode_paged.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32,
                                           i32, i32, i32, i32, i32, i32, f64]
    lib.fa_oracle_fwd_mod.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                      i32, i32, i32, f64, f64, P]
    lib.fa_oracle_set_threads.argtypes = [i32]
    for f in (lib.fa_oracle_set_threads, lib.fa_oracle_rows, lib.fa_oracle_fwd, lib.fa_oracle_varlen,
              lib.fa_oracle_decode, lib.fa_oracle_bwd, lib.fa_oracle_decode_paged,
              lib.fa_oracle_fwd_mod):
        f.restype = ctypes.c_int
    return lib


def load(path: str = LIB) -> ctypes.CDLL:
    """Load (building first if the shared object is missing) the oracle."""
    with _lock:
        if path in _lib_cache:
            return _lib_cache[path]
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        elif path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC):
            build()   # the source changed since the library was built
        lib = _bind(ctypes.CDLL(path))
        _lib_cache[path] = lib
        return lib


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous float64 numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _scale(scale, d: int) -> float:
    # Default scale 1/sqrt(d): "Checking correctness" on the FlashAttention
    # explainer page; softmax_scale=None on the skill page.
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def decode_e4m3(codes) -> np.ndarray:
    """fp64 values of 8-bit e4m3 codes (the OCP 8-bit floating-point format:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
    holds the subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN)."""
    try:
        import torch
        if isinstance(codes, torch.Tensor):
            codes = codes.detach().to("cpu").view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.ascontiguousarray(sign * mag)


class Oracle:
    """Thin marshalling wrapper around one loaded oracle shared object."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def set_threads(self, n: int) -> int:
        """OpenMP threads of the row loops (n < 1: unchanged); returns the count in effect."""
        return int(self.lib.fa_oracle_set_threads(int(n)))

    # -- padded batch ------------------------------------------------------
    def attention(self, q, k, v, causal=False, window=(-1, -1), scale=None):
        """q: [B,Sq,Hq,d]; k,v: [B,Sk,Hkv,d] -> (out [B,Sq,Hq,d], lse [B,Hq,Sq])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Sq, Hq, d = q.shape
        Bk, Sk, Hkv, dk = k.shape
        assert Bk == B and dk == d and v.shape == k.shape
        out = np.empty_like(q)
        lse = np.empty((B, Hq, Sq), dtype=np.float64)
        rc = self.lib.fa_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    B, Hq, Hkv, Sq, Sk, d, int(bool(causal)),
                                    int(window[0]), int(window[1]), _scale(scale, d))
        if rc != 0:
            raise RuntimeError(f"oracle fwd failed: {rc}")
        return out, lse

    # -- padded batch with score modifiers ------------------------------------
    def attention_mod(self, q, k, v, causal=False, window=(-1, -1), scale=None, softcap=0.0,
                      alibi_slopes=None):
        """As attention(), with soft-capping (cap * tanh(s / cap), 0 = off) and
        an ALiBi bias -slope_h * |pos_i - j| (alibi_slopes: [Hq] or None)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Sq, Hq, d = q.shape
        Bk, Sk, Hkv, dk = k.shape
        assert Bk == B and dk == d and v.shape == k.shape
        sl = None
        if alibi_slopes is not None:
            sl = _f64(alibi_slopes).reshape(-1)
            assert sl.shape == (Hq,)
        out = np.empty_like(q)
        lse = np.empty((B, Hq, Sq), dtype=np.float64)
        rc = self.lib.fa_oracle_fwd_mod(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        B, Hq, Hkv, Sq, Sk, d, int(bool(causal)),
                                        int(window[0]), int(window[1]), _scale(scale, d),
                                        float(softcap), _ptr(sl) if sl is not None else None)
        if rc != 0:
            raise RuntimeError(f"oracle fwd_mod failed: {rc}")
        return out, lse

    # -- 8-bit inputs ----------------------------------------------------------
    def attention_fp8(self, q8, k8, v8, descale_q, descale_k, descale_v, causal=False,
                      window=(-1, -1), scale=None):
        """Attention of 8-bit e4m3 inputs (uint8 codes, layouts as attention())
        whose real values are descale * decode(code): the values are decoded
        exactly (decode_e4m3) and scaled in fp64 (exact: a 4-bit significand
        times an fp32 factor), then the plain definition applies."""
        q = decode_e4m3(q8) * float(descale_q)
        k = decode_e4m3(k8) * float(descale_k)
        v = decode_e4m3(v8) * float(descale_v)
        d = q.shape[-1]
        return self.attention(q, k, v, causal=causal, window=window,
                              scale=_scale(scale, d))

    # -- gradients (padded batch) -------------------------------------------
    def attention_bwd(self, q, k, v, dout, causal=False, window=(-1, -1), scale=None):
        """q, dout: [B,Sq,Hq,d]; k,v: [B,Sk,Hkv,d] -> (dq, dk, dv) of the
        padded-batch attention for the incoming output gradient dout."""
        q, k, v, go = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Sq, Hq, d = q.shape
        Bk, Sk, Hkv, dk_ = k.shape
        assert Bk == B and dk_ == d and v.shape == k.shape and go.shape == q.shape
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(v)
        rc = self.lib.fa_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(go), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, Hq, Hkv, Sq, Sk, d, int(bool(causal)),
                                    int(window[0]), int(window[1]), _scale(scale, d))
        if rc != 0:
            raise RuntimeError(f"oracle bwd failed: {rc}")
        return dq, dk, dv

    # -- packed sequences --------------------------------------------------
    def attention_varlen(self, q, k, v, cu_q, cu_k, causal=False, window=(-1, -1),
                         scale=None):
        """q: [total_q,Hq,d]; k,v: [total_k,Hkv,d]; cu_*: [nseq+1]
        -> (out [total_q,Hq,d], lse [Hq,total_q])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        cu_q, cu_k = _i32(cu_q), _i32(cu_k)
        total_q, Hq, d = q.shape
        _, Hkv, _ = k.shape
        nseq = cu_q.shape[0] - 1
        assert cu_k.shape[0] == nseq + 1 and cu_q[-1] == total_q
        assert cu_k[-1] <= k.shape[0]
        out = np.empty_like(q)
        lse = np.empty((Hq, total_q), dtype=np.float64)
        rc = self.lib.fa_oracle_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                       _ptr(cu_q), _ptr(cu_k), nseq, Hq, Hkv, d,
                                       int(bool(causal)), int(window[0]), int(window[1]),
                                       _scale(scale, d))
        if rc != 0:
            raise RuntimeError(f"oracle varlen failed: {rc}")
        return out, lse

    # -- decode --------------------------------------------------------------
    def attention_decode(self, q, k_cache, v_cache, cache_seqlens, causal=False,
                         window=(-1, -1), scale=None):
        """q: [B,1,Hq,d]; caches: [B,Sk_cap,Hkv,d]; cache_seqlens: [B]
        -> (out [B,1,Hq,d], lse [B,Hq])."""
        q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
        sl = _i32(cache_seqlens)
        B, one, Hq, d = q.shape
        assert one == 1
        _, Sk_cap, Hkv, _ = kc.shape
        assert (sl >= 0).all() and (sl <= Sk_cap).all()
        out = np.empty_like(q)
        lse = np.empty((B, Hq), dtype=np.float64)
        rc = self.lib.fa_oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), _ptr(out),
                                       _ptr(lse), B, Hq, Hkv, Sk_cap, d, int(bool(causal)),
                                       int(window[0]), int(window[1]), _scale(scale, d))
        if rc != 0:
            raise RuntimeError(f"oracle decode failed: {rc}")
        return out, lse

    # -- decode against a paged cache, with an optional append ---------------
    def attention_decode_paged(self, q, k_pages, v_pages, block_table, cache_seqlens,
                               k_new=None, v_new=None, causal=False, window=(-1, -1),
                               scale=None):
        """q: [B,1,Hq,d]; pages: [num_pages,page_size,Hkv,d]; block_table:
        [B,max_pages]; cache_seqlens: [B] tokens in the cache; k_new, v_new:
        [B,1,Hkv,d] or None.  The caller's pages are not modified.
        -> (out [B,1,Hq,d], lse [B,Hq], k_pages', v_pages') where the primed
        pages hold the appended rows."""
        q = _f64(q)
        kp, vp = _f64(k_pages).copy(), _f64(v_pages).copy()
        bt, sl = _i32(block_table), _i32(cache_seqlens)
        B, one, Hq, d = q.shape
        assert one == 1
        num_pages, page_size, Hkv, _ = kp.shape
        assert bt.ndim == 2 and bt.shape[0] == B and sl.shape == (B,)
        kn = vn = None
        if k_new is not None:
            kn, vn = _f64(k_new), _f64(v_new)
            assert kn.shape == (B, 1, Hkv, d) and vn.shape == kn.shape
        out = np.empty_like(q)
        lse = np.empty((B, Hq), dtype=np.float64)
        rc = self.lib.fa_oracle_decode_paged(
            _ptr(q), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(sl),
            _ptr(kn) if kn is not None else None, _ptr(vn) if vn is not None else None,
            _ptr(out), _ptr(lse), B, Hq, Hkv, num_pages, page_size, bt.shape[1], d,
            int(bool(causal)), int(window[0]), int(window[1]), _scale(scale, d))
        if rc != 0:
            raise RuntimeError(f"oracle paged decode failed: {rc}")
        return out, lse, kp, vp

    # -- sampled rows of one (sequence, head) ------------------------------
    def attention_rows(self, q_rows, qi, sq, k_seq, v_seq, causal=False,
                       window=(-1, -1), scale=None):
        """q_rows: [n,d] query rows with indices qi[n] in a sequence of sq
        queries; k_seq, v_seq: [sk,d] of the matching K/V head.
        -> (out [n,d], lse [n])."""
        q, k, v = _f64(q_rows), _f64(k_seq), _f64(v_seq)
        qi = np.ascontiguousarray(np.asarray(qi, dtype=np.int64))
        n, d = q.shape
        sk = k.shape[0]
        out = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self.lib.fa_oracle_rows(_ptr(q), d, _ptr(qi), n, int(sq), _ptr(k), _ptr(v), d,
                                     sk, d, int(bool(causal)), int(window[0]),
                                     int(window[1]), _scale(scale, d), _ptr(out), d,
                                     _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"oracle rows failed: {rc}")
        return out, lse


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(*a, **kw):
    return default().attention(*a, **kw)


def attention_mod(*a, **kw):
    return default().attention_mod(*a, **kw)


def attention_varlen(*a, **kw):
    return default().attention_varlen(*a, **kw)


def attention_decode(*a, **kw):
    return default().attention_decode(*a, **kw)


def attention_decode_paged(*a, **kw):
    return default().attention_decode_paged(*a, **kw)


def attention_fp8(*a, **kw):
    return default().attention_fp8(*a, **kw)


def attention_bwd(*a, **kw):
    return default().attention_bwd(*a, **kw)


def attention_rows(*a, **kw):
    return default().attention_rows(*a, **kw)
