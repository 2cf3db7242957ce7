"""Checks on the gfx950 assembly of the pipelined kernels (CPU only: hipcc
cross-compiles, nothing runs on a GPU).

The forward and backward kernels feed their LDS rings with copies written in
inline asm and wait for them with hand-counted ``s_waitcnt vmcnt(N)``.  The
compiler does not see those copies, so two things it may do on its own would
break the pipelining without changing any result:

* place a ``vmcnt`` wait of its own inside a loop (for a load it issued
  before the loop, at that value's first use): the wait then runs on every
  step and drains every copy in flight;
* spill registers to scratch inside a loop: every reload is a vector-memory
  access that waits behind the copies.

Each kernel is compiled to assembly with the library's own flags and every
loop block is checked for both.  (The decode split kernel is not checked: it
loads V into registers with ordinary loads inside its loop by design and
counts them in its waits; the V-transpose pre-pass of the 8-bit forward has
no copy pipeline.)
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_08_amd import build_ext

PIPELINED = {
    "fa_fwd.hip": ("fa_fwd_kernel",),
    "fa_fwd_wide.hip": ("fa_fwd_wide_kernel",),
    "fa_fwd_fp8.hip": ("fa_fwd_fp8_kernel", "fa_fwd_fp8_paired_kernel"),
    "fa_bwd.hip": ("fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"),
}

_BLOCK = re.compile(r"^(\.LBB\w+|; %bb\.\d+):")
_KERNEL = re.compile(r"^(_ZN2fa\d+(\w+?)I\w*):")


def loop_findings(asm: str, kernel_names):
    """(kernel symbol, line, text) of every compiler-placed vmcnt wait and
    every scratch access inside a loop block of the named kernels."""
    found = []
    kernel = None
    in_asm = in_loop = False
    for n, line in enumerate(asm.splitlines(), 1):
        m = _KERNEL.match(line)
        if m:
            kernel = m.group(1) if m.group(2) in kernel_names else None
            in_loop = in_asm = False
            continue
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        if _BLOCK.match(line):
            in_loop = "Loop" in line
            continue
        if kernel is None or in_asm or not in_loop:
            continue
        text = line.strip()
        if (text.startswith("s_waitcnt") and "vmcnt" in text) or text.startswith("scratch_"):
            found.append((kernel, n, text))
    return found


def test_loop_finder_on_a_sample():
    # a wait inside a loop block is reported; one in an asm block, one
    # outside any loop and one in another kernel are not
    asm = "\n".join([
        "_ZN2fa13fa_fwd_kernelILi128EEEvNS_9FwdParamsE:",
        "\ts_waitcnt vmcnt(0)",
        ".LBB0_3:                               ; =>This Inner Loop Header: Depth=1",
        "\t;;#ASMSTART",
        "\ts_waitcnt vmcnt(4)",
        "\t;;#ASMEND",
        "\ts_waitcnt vmcnt(2) lgkmcnt(0)",
        "\tscratch_load_dwordx4 v[4:7], off, off",
        "; %bb.4:",
        "\ts_waitcnt vmcnt(0)",
        "_ZN2fa17fa_other_kernelILi128EEEvNS_9FwdParamsE:",
        ".LBB1_2:                               ;   in Loop: Header=BB1_2 Depth=1",
        "\ts_waitcnt vmcnt(0)",
    ])
    got = loop_findings(asm, ("fa_fwd_kernel",))
    assert [t for _, _, t in got] == ["s_waitcnt vmcnt(2) lgkmcnt(0)", "scratch_load_dwordx4 v[4:7], off, off"]


def _assembly(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [build_ext.HIPCC, *build_ext.FLAGS, *build_ext.EXTRA.get(src, []), "--offload-device-only", "-S",
           os.path.join(build_ext.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(shutil.which(build_ext.HIPCC) is None and not os.path.exists(build_ext.HIPCC),
                    reason="hipcc not available")
def test_no_compiler_wait_or_spill_inside_pipelined_loops(tmp_path):
    with ThreadPoolExecutor(max_workers=len(PIPELINED)) as ex:
        asm = dict(zip(PIPELINED, ex.map(lambda s: _assembly(s, str(tmp_path)), PIPELINED)))
    problems = []
    for src, names in PIPELINED.items():
        text = asm[src]
        for name in names:
            assert re.search(rf"^_ZN2fa\d+{name}I", text, re.M), f"{name} not found in {src}"
        problems += [f"{src}: {k} line {n}: {t}" for k, n, t in loop_findings(text, names)]
    assert not problems, "\n".join(problems[:20])
