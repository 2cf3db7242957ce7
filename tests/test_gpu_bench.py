"""bench.py's output contract, run end to end on the GPU with few steps:
one JSON line with the metric fields, the roofline object of the dominant
kernel and the CPU-oracle baseline (values only checked for sanity; the
timed numbers themselves come from the full-length run)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract():
    print("[case] bench.py --steps 3 --warmup 1 (forward leg only)", flush=True)
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-decode", "--no-backward", "--no-mods", "--no-fp8", "--no-configs",
           "--cpu-budget", "1"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"] == "causal_gqa_prefill" and d["dtype"] == "bf16"
    assert 0 < d["value"] < 2516.6 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2516.6
    assert 0 < rf["achieved"] < rf["peak"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    st = d["ms_per_call"]
    assert 0 < st["min"] <= st["median"] and st["mean"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["cpu_model"] and cb["single_thread"]["kvcache_decode"]["unit"] == "GB/s"


def test_bench_config_leg():
    """One other forward workload on its own (the HBM-bound sliding window):
    its roofline is judged against max(FLOP / MFMA peak, bytes / HBM peak)."""
    print("[case] bench.py --only-config causal_window", flush=True)
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--only-config", "causal_window"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    d = json.loads(lines[-1])
    rf = d["roofline"]
    assert d["workload"] == "causal_window" and rf["bound"] == "hbm" and rf["unit"] == "GB/s"
    assert 0 < rf["frac_of_roofline_time"] < 1 and rf["kernel"] == "fa_fwd_kernel"
