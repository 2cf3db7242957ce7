"""AddressSanitizer and UBSan runs of the host code (CPU only; GPU code is
never built with a sanitizer here):

  * the C-ABI source built with g++ -fsanitize=address,undefined against the
    recording stand-ins of tests/host_stub.cpp, driven through the ABI
    argument checks (test_abi_cpu.py) and the host-logic tests
    (test_host_stub.py);
  * the fp64 oracle (oracle/fa_oracle.c) built the same way, driven through
    all of its pins (test_oracle_pins.py).

Each run is a child Python process with the sanitizer runtime preloaded and
no recovery from a report, so any out-of-bounds access, use after free or
undefined behaviour fails the child and this test.  Leak detection is off
(the interpreter itself keeps memory until exit)."""
import os
import subprocess
import sys

import host_stub

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run_under_asan(tmp_path, tests, extra_env):
    env = dict(os.environ)
    env.update(extra_env)
    env["LD_PRELOAD"] = host_stub.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(HERE, t) for t in tests]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
    return out


def test_c_abi_under_asan_and_ubsan(tmp_path):
    lib = host_stub.build(str(tmp_path / "libfa_host_asan.so"), sanitize=True)
    out = _run_under_asan(tmp_path, ["test_abi_cpu.py", "test_host_stub.py"],
                          {"FA_TEST_LIB": lib, "FA_TEST_STUB_LIB": lib})
    print(out.strip().splitlines()[-1])


def test_oracle_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "libfa_oracle_asan.so"),
                       extra_flags=("-g", *host_stub.SANITIZE))
    out = _run_under_asan(tmp_path, ["test_oracle_pins.py"], {"FA_TEST_ORACLE_LIB": lib})
    print(out.strip().splitlines()[-1])
