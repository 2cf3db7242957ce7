"""Builds the C-ABI source (exact_attention_08_amd/csrc/fa_api.cpp) for the
host with g++, linked against host_stub.cpp in place of the kernels and the
HIP runtime, and binds the stub's recording calls.  The result exports every
fa_* symbol of include/fa.h, so exact_attention_08_amd.fa can load it in
place of the GPU library; any call that passes the host checks "launches" a
recording stand-in instead of a kernel.  Used by the host-logic and
sanitizer tests (CPU only)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "exact_attention_08_amd", "csrc")
SOURCES = [os.path.join(CSRC, "fa_api.cpp"), os.path.join(HERE, "host_stub.cpp")]
SANITIZE = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer")

FWD_FIELDS = ["d", "bf16", "varlen", "B", "Hq", "Hkv", "G", "Sq", "Sk", "nqt", "q_tok_stride",
              "kv_tok_stride", "lse_b_stride", "lse_h_stride", "causal", "wl", "wr", "qsign",
              "xcd_groups", "gw", "bm", "mod", "alibi", "cu_q", "cu_k", "lse"]
FP8_FIELDS = ["B", "Hq", "Hkv", "G", "Sq", "Sk", "sk_pad", "nqt", "causal", "wl", "wr", "qsign",
              "xcd_groups", "gw", "bm", "vt"]
DECODE_FIELDS = ["d", "bf16", "B", "Hq", "Hkv", "G", "Sk_cap", "max_len", "nsplit", "split",
                 "qblocks", "causal", "wl", "wr", "qsign", "page_size", "max_pages",
                 "num_pages", "append", "ws_o", "ws_lse", "block_table", "k_new", "v_new"]
BWD_FIELDS = ["d", "bf16", "B", "Hq", "Hkv", "G", "Sq", "Sk", "q_tok_stride", "kv_tok_stride",
              "causal", "wl", "wr", "nkb", "gw", "nqb", "dsum", "lse2"]


def asan_runtime() -> str:
    """gcc's AddressSanitizer runtime, which must be preloaded into Python."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build(out: str, sanitize: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           *(SANITIZE if sanitize else ()), "-o", out, *SOURCES]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


class Stub:
    """The stub's recording calls on a loaded host build."""

    def __init__(self, lib: ctypes.CDLL):
        self.lib = lib
        lib.fa_stub_set.argtypes = [ctypes.c_int] * 4
        lib.fa_stub_kernel.restype = ctypes.c_char_p
        lib.fa_stub_scratch_address.restype = ctypes.c_longlong
        for name in ("fwd_c", "fwd_sc_k", "fwd_sc_c", "fp8_c", "fp8_descale_v", "decode_c",
                     "bwd_scale", "bwd_c2"):
            getattr(lib, "fa_stub_" + name).restype = ctypes.c_float

    def set(self, launch_error=0, device_error=0, stream_device=0, scratch_error=0):
        self.lib.fa_stub_set(launch_error, device_error, stream_device, scratch_error)
        self.lib.fa_stub_reset()

    @property
    def calls(self) -> int:
        return int(self.lib.fa_stub_calls())

    @property
    def kernel(self) -> str:
        return self.lib.fa_stub_kernel().decode()

    @property
    def scratch_address(self) -> int:
        return int(self.lib.fa_stub_scratch_address())

    def _fields(self, fn, names):
        buf = (ctypes.c_longlong * len(names))()
        fn(buf)
        return dict(zip(names, buf))

    def fwd(self):
        f = self._fields(self.lib.fa_stub_fwd, FWD_FIELDS)
        f.update(c=self.lib.fa_stub_fwd_c(), sc_k=self.lib.fa_stub_fwd_sc_k(),
                 sc_c=self.lib.fa_stub_fwd_sc_c())
        return f

    def fp8(self):
        f = self._fields(self.lib.fa_stub_fp8, FP8_FIELDS)
        f.update(c=self.lib.fa_stub_fp8_c(), descale_v=self.lib.fa_stub_fp8_descale_v())
        return f

    def decode(self):
        f = self._fields(self.lib.fa_stub_decode, DECODE_FIELDS)
        f.update(c=self.lib.fa_stub_decode_c())
        return f

    def bwd(self):
        f = self._fields(self.lib.fa_stub_bwd, BWD_FIELDS)
        f.update(scale=self.lib.fa_stub_bwd_scale(), c2=self.lib.fa_stub_bwd_c2())
        return f
