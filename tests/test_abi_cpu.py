"""The C-ABI library on the CPU: it loads, exports every symbol include/fa.h
declares, and rejects bad arguments on the host before any HIP call (so no
GPU is needed; no compute call is made)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 0x10000          # 16-byte aligned, never dereferenced by a rejected call
MISALIGNED = 0x10002


@pytest.fixture(scope="module")
def lib():
    from exact_attention_08_amd import fa
    if os.environ.get("FA_TEST_LIB"):       # a host build (the sanitizer run)
        return fa.load(os.environ["FA_TEST_LIB"])
    if not os.path.exists(fa.LIB_PATH):
        from exact_attention_08_amd import build_ext
        build_ext.build()
    return fa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(["fa_fwd", "fa_fwd_mod", "fa_fwd_fp8_workspace_bytes",
                                           "fa_fwd_fp8", "fa_fwd_varlen",
                                           "fa_decode_workspace_bytes",
                                           "fa_decode_kvcache", "fa_decode_kvcache_noalloc",
                                           "fa_decode_paged",
                                           "fa_bwd_workspace_bytes", "fa_bwd", "fa_status_str",
                                           "fa_last_error"])


def test_every_declared_symbol_is_exported(lib):
    from exact_attention_08_amd import fa
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(fa.EXPORTS) == set(declared_functions())


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128,
        causal=0, wl=-1, wr=-1, scale=0.125, dtype=0):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, wl, wr, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(q=None, Sk=0), 1), (dict(o=None, Sk=0), 1),
    (dict(q=MISALIGNED), 1), (dict(o=MISALIGNED), 1), (dict(lse=FAKE + 2), 1),
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(wl=-2), 1), (dict(wr=-5), 1), (dict(scale=math.nan), 1), (dict(scale=math.inf), 1),
    (dict(Sq=-1), 1), (dict(Sk=-3), 1),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""
    assert lib.fa_status_str(status).decode().startswith("FA_ERR_")


def test_fwd_null_kv_allowed_only_without_keys(lib):
    assert fwd(lib, k=None, Sk=5) == 1
    assert fwd(lib, v=None, Sk=5) == 1
    # with Sk == 0 a null k/v passes validation; Sq == 0 keeps the call a no-op
    assert fwd(lib, k=None, v=None, Sk=0, Sq=0) == 0


def test_fwd_empty_query_is_a_noop(lib):
    # Sq == 0 returns before any HIP call, with nothing enqueued
    assert fwd(lib, Sq=0) == 0
    assert lib.fa_last_error().decode() == ""


def fwd_mod(lib, alibi=None, softcap=0.0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128,
             causal=0, wl=-1, wr=-1, scale=0.125, dtype=0)
    a.update(kw)
    return lib.fa_fwd_mod(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Sk"], a["d"], a["causal"], a["wl"], a["wr"], a["scale"],
                          alibi, softcap, a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(softcap=-1.0), 1), (dict(softcap=math.nan), 1), (dict(softcap=math.inf), 1),
    (dict(alibi=FAKE + 2), 1), (dict(alibi=FAKE, q=None), 1), (dict(softcap=5.0, d=96), 2),
    (dict(alibi=FAKE, Hq=6, Hkv=4), 1), (dict(softcap=2.0, scale=math.inf), 1),
    (dict(q=None), 1),    # no modifier: the plain forward's checks
])
def test_fwd_mod_rejects(lib, kw, status):
    assert fwd_mod(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_fwd_mod_empty_query_is_a_noop(lib):
    assert fwd_mod(lib, alibi=FAKE, softcap=3.0, Sq=0) == 0


def fp8(lib, ws=FAKE, ws_bytes=1 << 30, dq=0.01, dk=0.01, dv=0.01, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128,
             causal=1, wl=-1, wr=-1, scale=0.125)
    a.update(kw)
    return lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Sk"], a["d"], a["causal"], a["wl"], a["wr"], a["scale"], dq,
                          dk, dv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=MISALIGNED), 1), (dict(dq=0.0), 1), (dict(dk=-1.0), 1),
    (dict(dv=math.nan), 1), (dict(dq=math.inf), 1), (dict(d=96), 2), (dict(Hq=6, Hkv=4), 1),
    (dict(ws=None), 3), (dict(ws=FAKE + 8), 3), (dict(ws_bytes=1 * 2 * 128 * 64 - 1), 3),
    (dict(scale=math.nan), 1), (dict(wl=-3), 1),
])
def test_fp8_rejects(lib, kw, status):
    assert fp8(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_fp8_workspace_bytes(lib):
    f = lib.fa_fwd_fp8_workspace_bytes
    assert f(4, 8, 4096, 128) == 4 * 8 * 128 * 4096
    assert f(1, 2, 65, 64) == 2 * 64 * 128
    assert f(1, 2, 0, 64) == 0
    assert fp8(lib, Sq=0) == 0


def varlen(lib, cu_q=FAKE, cu_k=FAKE, B=2, maxq=8, maxk=8, total_q=10, d=128, **kw):
    return lib.fa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, cu_q, cu_k, B, 4, 2, maxq, maxk,
                             total_q, d, 1, -1, -1, 0.1, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu_q=None), 1), (dict(cu_k=None), 1), (dict(cu_q=FAKE + 1), 1), (dict(maxq=-1), 1),
    (dict(total_q=-1), 1), (dict(d=80), 2),
])
def test_varlen_rejects(lib, kw, status):
    assert varlen(lib, **kw) == status


def test_varlen_empty_is_a_noop(lib):
    assert varlen(lib, total_q=0) == 0
    assert varlen(lib, maxq=0) == 0


def test_workspace_bytes(lib):
    f = lib.fa_decode_workspace_bytes
    assert f(64, 32, 32768, 128, 1024) == 64 * 32 * 32 * 129 * 4
    assert f(3, 5, 1000, 64, 256) == 3 * 5 * 4 * 65 * 4
    assert f(1, 1, 1, 128, 1024) == 129 * 4
    assert f(0, 1, 1, 128, 1024) == 0


def decode(lib, ws=FAKE, ws_bytes=1 << 30, B=2, Hq=8, Hkv=2, cap=4096, maxk=4096, d=128,
           split=1024, seqlens=FAKE, dtype=0):
    return lib.fa_decode_kvcache(FAKE, FAKE, FAKE, seqlens, FAKE, FAKE, B, Hq, Hkv, cap, maxk, d,
                                 1, -1, -1, 0.1, split, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), 3), (dict(ws=FAKE + 8), 3), (dict(ws_bytes=1000), 3),
    (dict(seqlens=None), 1), (dict(cap=0), 1), (dict(maxk=0), 1), (dict(maxk=5000), 1),
    (dict(split=100), 1), (dict(split=0), 1), (dict(d=32), 2), (dict(Hq=7), 1), (dict(dtype=3), 2),
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def test_workspace_exact_boundary(lib):
    need = lib.fa_decode_workspace_bytes(2, 8, 4096, 128, 1024)
    assert decode(lib, ws_bytes=need - 1) == 3
    assert "workspace too small" in lib.fa_last_error().decode()


def decode_noalloc(lib, B=2, Hq=8, Hkv=2, cap=4096, maxk=4096, d=128, split=1024,
                   seqlens=FAKE, dtype=0):
    return lib.fa_decode_kvcache_noalloc(FAKE, FAKE, FAKE, seqlens, FAKE, FAKE, B, Hq, Hkv, cap,
                                         maxk, d, 1, -1, -1, 0.1, split, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(seqlens=None), 1), (dict(cap=0), 1), (dict(maxk=0), 1), (dict(maxk=5000), 1),
    (dict(split=100), 1), (dict(d=32), 2), (dict(Hq=7), 1), (dict(dtype=3), 2),
    # partials beyond the 64 MiB scratch array: 64 x 32 x 64 splits x 129 x 4 B
    (dict(B=64, Hq=32, Hkv=8, cap=65536, maxk=65536), 3),
])
def test_decode_noalloc_rejects_on_the_host(lib, kw, status):
    assert decode_noalloc(lib, **kw) == status
    if status == 3:
        assert "scratch" in lib.fa_last_error().decode()


def test_decode_noalloc_limit_matches_header(lib):
    from exact_attention_08_amd import fa
    text = open(HEADER).read()
    assert "#define FA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)" in text
    assert fa.DECODE_NOALLOC_MAX_BYTES == 64 << 20
    # the largest benchmark decode (64 x 32 heads, 32768 keys, 1024-key splits) fits
    assert lib.fa_decode_workspace_bytes(64, 32, 32768, 128, 1024) <= fa.DECODE_NOALLOC_MAX_BYTES


def paged(lib, kp=FAKE, table=FAKE, seqlens=FAKE, kn=None, vn=None, ws=FAKE, ws_bytes=1 << 30,
          B=2, Hq=8, Hkv=2, num_pages=16, page=256, max_pages=8, maxk=2048, d=128, split=1024,
          dtype=0):
    return lib.fa_decode_paged(FAKE, kp, FAKE, table, seqlens, kn, vn, FAKE, FAKE, B, Hq, Hkv,
                               num_pages, page, max_pages, maxk, d, 1, -1, -1, 0.1, split, ws,
                               ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kp=None), 1), (dict(table=None), 1), (dict(table=FAKE + 2), 1), (dict(seqlens=None), 1),
    (dict(kn=FAKE), 1), (dict(vn=FAKE), 1), (dict(kn=FAKE + 8, vn=FAKE), 1),
    (dict(page=16), 1), (dict(page=48), 1), (dict(page=0), 1), (dict(num_pages=0), 1),
    (dict(max_pages=0), 1), (dict(maxk=0), 1), (dict(maxk=8 * 256 + 1), 1), (dict(split=32), 1),
    (dict(ws=None), 3), (dict(ws_bytes=1000), 3), (dict(d=96), 2), (dict(dtype=2), 2),
    (dict(Hq=7), 1),
])
def test_paged_rejects(lib, kw, status):
    assert paged(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_paged_workspace_exact_boundary(lib):
    need = lib.fa_decode_workspace_bytes(2, 8, 2048, 128, 1024)
    assert paged(lib, ws_bytes=need - 1) == 3
    assert "workspace too small" in lib.fa_last_error().decode()


def bwd(lib, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, ws_bytes=1 << 30, B=1,
        Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.125, dtype=0):
    return lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, 1, -1,
                      -1, scale, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dout=None), 1), (dict(dout=MISALIGNED), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=MISALIGNED), 1), (dict(lse=None), 1), (dict(ws=None), 3), (dict(ws=FAKE + 8), 3),
    (dict(ws_bytes=4 * 8 * 4 - 1, B=1, Hq=4, Sq=8), 3), (dict(d=80), 2), (dict(dtype=5), 2),
    (dict(Hq=6, Hkv=4), 1), (dict(scale=math.nan), 1), (dict(Sq=-2), 1),
])
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status
    assert lib.fa_last_error().decode() != ""


def test_bwd_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(4, 32, 4096) == 2 * 4 * 32 * 4096 * 4
    assert lib.fa_bwd_workspace_bytes(0, 32, 4096) == 0


def test_bwd_empty_is_a_noop(lib):
    # no queries and no keys: nothing to write, nothing enqueued
    assert bwd(lib, Sq=0, Sk=0, ws=None, ws_bytes=0) == 0
    assert lib.fa_last_error().decode() == ""


def test_status_strings(lib):
    names = ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP"]
    for i, n in enumerate(names):
        assert lib.fa_status_str(i).decode() == n


def test_binding_fails_loudly_without_library(tmp_path):
    from exact_attention_08_amd import fa
    with pytest.raises(RuntimeError, match="not built"):
        fa.load(str(tmp_path / "missing.so"))
    # calls routed to a missing library raise too (no fallback)
    with pytest.raises(RuntimeError, match="not built"):
        with fa.using(str(tmp_path / "missing.so")):
            pass


def test_checking_library_exports_the_same_symbols(lib):
    """The checking build (libfa355_debug.so) exports every declared entry
    point, like the pipelined library."""
    from exact_attention_08_amd import fa
    assert os.path.exists(fa.DEBUG_LIB_PATH)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.DEBUG_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_package_exports_a_binding_for_every_entry_point():
    import exact_attention_08_amd as pkg
    for name in declared_functions():
        if name in ("fa_status_str", "fa_last_error"):
            continue                      # surfaced through FAError
        py = name[len("fa_"):]
        assert py in pkg.__all__ and callable(getattr(pkg, py)), py
