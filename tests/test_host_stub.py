"""Host logic of the C ABI with the kernels replaced by recording stand-ins
(tests/host_stub.cpp): which forward kernel a call chooses, the parameter
blocks the launchers receive (tile counts, strides, scale constants,
workspace carving), the FA_ERR_HIP path of a failed launch, and the device
checks of the allocation-free decode.  CPU only: the library is the C-ABI
source built with g++ against the stand-ins, so no GPU or HIP runtime is
involved.  FA_TEST_STUB_LIB names a prebuilt host library (the sanitizer
test runs this module against one built with AddressSanitizer and UBSan)."""
import math
import os

import pytest

import host_stub

FAKE = 0x10000
OTHER = 0x20000
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
LOG2E = 1.4426950408889634
FLT_MIN = 1.17549435e-38


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    from exact_attention_08_amd import fa
    path = os.environ.get("FA_TEST_STUB_LIB")
    if not path:
        path = host_stub.build(str(tmp_path_factory.mktemp("stub") / "libfa_host_stub.so"))
    return fa.load(path)


@pytest.fixture
def stub(lib):
    s = host_stub.Stub(lib)
    s.set()
    yield s
    s.set()


def _f32(x):
    import numpy as np
    return float(np.float32(x))


def fwd(lib, B=1, Hq=8, Hkv=2, Sq=256, Sk=256, d=128, causal=1, wl=-1, wr=-1, scale=0.125,
        dtype=0, lse=FAKE, stream=None):
    return lib.fa_fwd(FAKE, FAKE, FAKE, FAKE, lse, B, Hq, Hkv, Sq, Sk, d, causal, wl, wr, scale,
                      dtype, stream)


# Sq, Sk, causal, wl, wr -> kernel: the paired kernel while a row sees at
# most 2560 keys on average (causal: Sk - min(Sq, Sk)/2; a left window bounds
# a row by wl + 1 (+ wr without causal)), the wide kernel beyond
DISPATCH = [
    (4096, 4096, 1, -1, -1, "paired"),
    (5120, 5120, 1, -1, -1, "paired"),         # 5120 - 2560 = 2560
    (5122, 5122, 1, -1, -1, "wide"),           # 5122 - 2561 = 2561
    (64, 2592, 1, -1, -1, "paired"),           # 2592 - 32
    (64, 2594, 1, -1, -1, "wide"),
    (8000, 2700, 1, -1, -1, "paired"),         # Sq > Sk: 2700 - 1350
    (64, 2560, 0, -1, -1, "paired"),
    (64, 2561, 0, -1, -1, "wide"),
    (4096, 8192, 1, 1000, -1, "paired"),
    (4096, 8192, 1, 2559, -1, "paired"),
    (4096, 8192, 1, 2560, -1, "wide"),
    (4096, 8192, 0, 1000, 1559, "paired"),
    (4096, 8192, 0, 1000, 1560, "wide"),
    (4096, 8192, 0, 1000, -1, "wide"),        # no right bound: rows see up to 8192 keys
    (4096, 8192, 0, -1, 1000, "wide"),
]


@pytest.mark.parametrize("Sq,Sk,causal,wl,wr,kernel", DISPATCH)
def test_forward_kernel_choice(lib, stub, Sq, Sk, causal, wl, wr, kernel):
    assert fwd(lib, Sq=Sq, Sk=Sk, causal=causal, wl=wl, wr=wr) == FA_OK
    assert stub.calls == 1 and stub.kernel == kernel
    p = stub.fwd()
    assert (p["wl"], p["wr"], p["causal"], p["varlen"]) == (wl, wr, causal, 0)


def test_window_that_cuts_no_row_is_dropped(lib, stub):
    # rows sit at key positions Sk - Sq .. Sk - 1: a left bound >= Sk - 1 and
    # a right bound >= Sq - 1 exclude no key of any row
    assert fwd(lib, Sq=4096, Sk=4096, wl=4095, wr=4095, causal=0) == FA_OK
    p = stub.fwd()
    assert (p["wl"], p["wr"]) == (-1, -1) and stub.kernel == "wide"
    assert fwd(lib, Sq=100, Sk=3000, wl=2998, wr=98, causal=0) == FA_OK
    p = stub.fwd()
    assert (p["wl"], p["wr"]) == (2998, 98)
    assert fwd(lib, Sq=100, Sk=3000, wl=2999, wr=99, causal=0) == FA_OK
    assert (stub.fwd()["wl"], stub.fwd()["wr"]) == (-1, -1)


# Hq, Hkv -> heads per work-group gw; rows per work-group = wave rows x 4 / gw
@pytest.mark.parametrize("Hq,Hkv,gw", [(8, 2, 4), (8, 8, 1), (12, 2, 2), (6, 2, 1), (32, 4, 4)])
@pytest.mark.parametrize("Sk,wave_rows", [(1000, 32), (4000, 64)])
def test_forward_tiles_and_strides(lib, stub, Hq, Hkv, gw, Sk, wave_rows):
    B, Sq, d = 3, 1000, 64
    assert fwd(lib, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, d=d) == FA_OK
    p = stub.fwd()
    bm = wave_rows * 4 // gw
    assert (p["G"], p["gw"], p["bm"], p["nqt"]) == (Hq // Hkv, gw, bm, -(-Sq // bm))
    assert (p["q_tok_stride"], p["kv_tok_stride"]) == (Hq * d, Hkv * d)
    assert (p["lse_b_stride"], p["lse_h_stride"]) == (Hq * Sq, Sq)
    assert p["d"] == d and p["bf16"] == 1
    assert p["xcd_groups"] == ((B * Hkv) // 8 if (B * Hkv) % 8 == 0 else 0)


def test_forward_xcd_groups(lib, stub):
    assert fwd(lib, B=4, Hq=8, Hkv=2) == FA_OK
    assert stub.fwd()["xcd_groups"] == 1
    assert fwd(lib, B=16, Hq=32, Hkv=8) == FA_OK
    assert stub.fwd()["xcd_groups"] == 16
    assert fwd(lib, B=3, Hq=8, Hkv=2) == FA_OK
    assert stub.fwd()["xcd_groups"] == 0


@pytest.mark.parametrize("scale,c,qsign", [
    (0.125, _f32(0.125 * LOG2E), 0),
    (-0.125, _f32(0.125 * LOG2E), 0x80008000),
    (0.0, FLT_MIN, 0),
])
def test_forward_scale_constants(lib, stub, scale, c, qsign):
    assert fwd(lib, scale=scale) == FA_OK
    p = stub.fwd()
    assert p["qsign"] == qsign
    assert math.isclose(p["c"], c, rel_tol=2 ** -22)


def test_fp16_and_lse_pointer(lib, stub):
    assert fwd(lib, dtype=1, lse=None) == FA_OK
    p = stub.fwd()
    assert p["bf16"] == 0 and p["lse"] == 0


def test_fwd_mod_kernel_choice_and_constants(lib, stub):
    st = lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 300, 300, 128, 1, -1, -1, 0.1,
                        OTHER, 30.0, 0, None)
    assert st == FA_OK and stub.kernel == "paired"
    p = stub.fwd()
    assert p["mod"] == 3 and p["alibi"] == OTHER and p["bm"] == 32
    assert math.isclose(p["sc_k"], 2 * 0.1 * LOG2E / 30.0, rel_tol=2 ** -22)
    assert math.isclose(p["sc_c"], 30.0 * LOG2E, rel_tol=2 ** -22)
    # rows that see more than 2560 keys on average: the wide kernel
    assert lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 6000, 6000, 128, 1, -1, -1, 0.1,
                          OTHER, 30.0, 0, None) == FA_OK
    assert stub.kernel == "wide" and stub.fwd()["mod"] == 3 and stub.fwd()["bm"] == 64
    # soft-capping alone, ALiBi alone
    assert lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 300, 300, 128, 1, -1, -1, 0.1,
                          None, 5.0, 0, None) == FA_OK
    assert stub.fwd()["mod"] == 2 and stub.fwd()["alibi"] == 0
    assert lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 300, 300, 128, 1, -1, -1, 0.1,
                          OTHER, 0.0, 0, None) == FA_OK
    assert stub.fwd()["mod"] == 1
    # no modifier: the plain forward
    assert lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 300, 300, 128, 1, -1, -1, 0.1,
                          None, 0.0, 0, None) == FA_OK
    assert stub.kernel == "paired" and stub.fwd()["mod"] == 0


@pytest.mark.parametrize("maxq,maxk,kernel", [(1500, 2048, "paired"), (5120, 5120, "paired"),
                                               (5200, 5200, "wide")])
def test_varlen_params(lib, stub, maxq, maxk, kernel):
    st = lib.fa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, OTHER, 5, 16, 4, maxq, maxk, 7000,
                           128, 1, -1, -1, 0.1, 0, None)
    assert st == FA_OK and stub.kernel == kernel
    p = stub.fwd()
    bm = (32 if kernel == "paired" else 64) * 4 // 4
    assert p["varlen"] == 1 and (p["cu_q"], p["cu_k"]) == (FAKE, OTHER)
    assert (p["Sq"], p["Sk"], p["nqt"]) == (maxq, maxk, -(-maxq // bm))
    assert (p["lse_b_stride"], p["lse_h_stride"]) == (0, 7000)


def test_fp8_params(lib, stub):
    st = lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 300, 333, 128, 1, -1, -1, -0.1,
                        0.5, 0.25, 2.0, OTHER, 1 << 20, None)
    assert st == FA_OK and stub.kernel == "fp8_paired"
    p = stub.fp8()
    assert (p["sk_pad"], p["vt"], p["bm"], p["nqt"]) == (384, OTHER, 32, 10)
    assert p["qsign"] == 0x80808080 and p["descale_v"] == 2.0
    assert math.isclose(p["c"], 0.1 * 0.5 * 0.25 * LOG2E, rel_tol=2 ** -21)
    # rows that see more than 2560 keys on average: the wide form
    stub.set()
    assert lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 6000, 6000, 128, 1, -1, -1, 0.1,
                          0.5, 0.25, 2.0, OTHER, 1 << 30, None) == FA_OK
    assert stub.kernel == "fp8_wide" and (stub.fp8()["bm"], stub.fp8()["nqt"]) == (64, 94)
    need = lib.fa_fwd_fp8_workspace_bytes(2, 2, 333, 128)
    assert need == 2 * 2 * 128 * 384
    stub.set()
    assert lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 300, 333, 128, 1, -1, -1, 0.1,
                          0.5, 0.25, 2.0, OTHER, need - 1, None) == FA_ERR_WORKSPACE
    assert stub.calls == 0


def test_decode_params(lib, stub):
    B, Hq, Hkv, d, maxk, split = 3, 40, 2, 128, 5000, 1024
    st = lib.fa_decode_kvcache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, 8192, maxk, d, 1,
                               -1, -1, 0.1, split, OTHER, 1 << 30, 0, None)
    assert st == FA_OK and stub.kernel == "decode"
    p = stub.decode()
    assert (p["G"], p["qblocks"], p["nsplit"], p["split"]) == (20, 2, 5, 1024)
    assert (p["Sk_cap"], p["max_len"], p["block_table"], p["append"]) == (8192, maxk, 0, 0)
    assert p["ws_o"] == OTHER and p["ws_lse"] == OTHER + B * Hq * 5 * d * 4
    assert lib.fa_decode_workspace_bytes(B, Hq, maxk, d, split) == B * Hq * 5 * (d + 1) * 4


def test_paged_params(lib, stub):
    st = lib.fa_decode_paged(FAKE, FAKE, FAKE, OTHER, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64,
                             128, 10, 1200, 64, 1, -1, -1, 0.1, 256, OTHER, 1 << 30, 1, None)
    assert st == FA_OK and stub.kernel == "paged"
    p = stub.decode()
    assert (p["page_size"], p["max_pages"], p["num_pages"], p["append"]) == (128, 10, 64, 1)
    assert (p["block_table"], p["k_new"], p["v_new"]) == (OTHER, FAKE, FAKE)
    assert (p["nsplit"], p["qblocks"], p["d"], p["bf16"]) == (5, 1, 64, 0)
    assert p["ws_lse"] == OTHER + 2 * 8 * 5 * 64 * 4


def test_bwd_params(lib, stub):
    B, Hq, Hkv, Sq, Sk = 2, 8, 2, 300, 333
    st = lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, Sq, Sk, 128,
                    1, -1, -1, -0.1, OTHER, 1 << 30, 0, None)
    assert st == FA_OK and stub.kernel == "bwd"
    p = stub.bwd()
    assert (p["nkb"], p["gw"], p["nqb"]) == (2, 4, -(-Sq // (32 * 8 // 4)))
    assert (p["dsum"], p["lse2"]) == (OTHER, OTHER + B * Hq * Sq * 4)
    assert p["scale"] == _f32(-0.1) and math.isclose(p["c2"], -0.1 * LOG2E, rel_tol=2 ** -22)
    assert lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, Sq, Sk,
                      64, 1, -1, -1, 0.1, OTHER, 1 << 30, 0, None) == FA_OK
    assert stub.bwd()["nqb"] == -(-Sq // (32 * 4 // 4))


def _every_entry_point(lib):
    """One valid call of each launching entry point."""
    return {
        "fa_fwd": lambda: fwd(lib),
        "fa_fwd_mod": lambda: lib.fa_fwd_mod(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64, 128, 1,
                                             -1, -1, 0.1, OTHER, 0.0, 0, None),
        "fa_fwd_varlen": lambda: lib.fa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8,
                                                   2, 64, 64, 100, 128, 1, -1, -1, 0.1, 0, None),
        "fa_fwd_fp8": lambda: lib.fa_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64, 128, 1,
                                             -1, -1, 0.1, 1.0, 1.0, 1.0, OTHER, 1 << 20, None),
        "fa_decode_kvcache": lambda: lib.fa_decode_kvcache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8,
                                                           2, 512, 512, 128, 1, -1, -1, 0.1, 256,
                                                           OTHER, 1 << 20, 0, None),
        "fa_decode_kvcache_noalloc": lambda: lib.fa_decode_kvcache_noalloc(
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 512, 512, 128, 1, -1, -1, 0.1, 256, 0,
            None),
        "fa_decode_paged": lambda: lib.fa_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                                       FAKE, FAKE, 2, 8, 2, 8, 64, 4, 256, 128, 1,
                                                       -1, -1, 0.1, 256, OTHER, 1 << 20, 0, None),
        "fa_bwd": lambda: lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2,
                                     64, 64, 128, 1, -1, -1, 0.1, OTHER, 1 << 20, 0, None),
    }


@pytest.mark.parametrize("name", list(_every_entry_point(None)))
def test_failed_launch_returns_fa_err_hip(lib, stub, name):
    call = _every_entry_point(lib)[name]
    stub.set(launch_error=98)
    assert call() == FA_ERR_HIP
    assert stub.calls == 1
    assert lib.fa_last_error().decode() == "kernel launch failed: stub HIP error 98"
    assert lib.fa_status_str(FA_ERR_HIP).decode() == "FA_ERR_HIP"
    # the next successful call clears the message
    stub.set()
    assert call() == FA_OK and lib.fa_last_error().decode() == ""


def test_noalloc_decode_uses_the_scratch_array(lib, stub):
    st = lib.fa_decode_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 8, 32768, 32768,
                                       128, 1, -1, -1, 0.1, 1024, 0, FAKE)
    assert st == FA_OK and stub.kernel == "decode"
    p = stub.decode()
    assert p["ws_o"] == stub.scratch_address
    assert p["ws_lse"] == stub.scratch_address + 4 * 32 * 32 * 128 * 4


def test_noalloc_decode_device_checks(lib, stub):
    def call(stream=None):
        return lib.fa_decode_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 512, 512,
                                             128, 1, -1, -1, 0.1, 256, 0, stream)
    stub.set(device_error=100)
    assert call() == FA_ERR_HIP and stub.calls == 0
    assert lib.fa_last_error().decode() == "device query failed: stub HIP error 100"
    stub.set(stream_device=1)
    assert call(FAKE) == FA_ERR_INVALID_ARG and stub.calls == 0
    assert "device 1" in lib.fa_last_error().decode()
    stub.set(stream_device=1)
    assert call(None) == FA_OK       # the null stream is the current device's
    stub.set(scratch_error=101)
    assert call() == FA_ERR_HIP and stub.calls == 0
    assert lib.fa_last_error().decode() == "scratch address lookup failed: stub HIP error 101"


@pytest.mark.parametrize("call", [
    lambda lib: fwd(lib, d=96),
    lambda lib: fwd(lib, Hq=7),
    lambda lib: fwd(lib, scale=math.nan),
    lambda lib: fwd(lib, B=1, Hq=1, Hkv=1, Sq=1 << 30, Sk=8),          # > 2 GiB per sequence
    lambda lib: fwd(lib, B=1 << 20, Hq=64, Hkv=64, Sq=1 << 16, Sk=8),  # grid too large
    lambda lib: lib.fa_decode_kvcache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 512, 512, 128,
                                      1, -1, -1, 0.1, 256, OTHER, 100, 0, None),
    lambda lib: lib.fa_decode_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 32, 8, 65536,
                                              65536, 128, 1, -1, -1, 0.1, 1024, 0, None),
    lambda lib: lib.fa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 64,
                           128, 1, -1, -1, 0.1, OTHER, 10, 0, None),
])
def test_rejected_calls_launch_nothing(lib, stub, call):
    assert call(lib) != FA_OK
    assert stub.calls == 0 and lib.fa_last_error().decode() != ""
