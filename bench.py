#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

A step is one call of the hot path on the headline workload: causal GQA
prefill, B=4, Hq=32, Hkv=8, S=4096, d=128, bf16 (one fa_fwd launch).  The
line's value, roofline and cpu_baseline are for that workload.  Beside it,
each with its own timing and roofline object:
  * "configs": the forward on the other workloads of the benchmark list --
    small non-causal (B=1, H=1, S=256, d=64), causal sliding window (B=2,
    H=32, S=16384, window (256, 256), fp16; bound by HBM, judged against
    max(FLOP / MFMA peak, bytes / HBM peak)), packed causal sequences (64
    lengths U{32..2048}, Hq=32, Hkv=8) and the 65,536-token causal prefill;
  * "decode": the KV-cache decode (B=64, Hq=32, Hkv=8, d=128, cache lengths
    U{1024..32768}, split 1024 + combine), and "decode_paged": the same keys
    in a shuffled pool of 256-row pages with each sequence's last key
    appended by the call (append, split, combine);
  * "forward_modifiers" (ALiBi and/or soft-capping), "forward_fp8" (e4m3
    inputs) and "backward" (fa_bwd) on the headline workload's shape.
Inputs are seeded synthetic tensors already resident in HBM.  Every timed
call is bracketed by events on the launch stream: ms per call is reported as
mean (the timed region over K calls), median and minimum.

Prints ONE JSON line.  --gpus N with N > 1 is refused: this build runs on one
GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from exact_attention_08_amd import fa, metrics, synth  # noqa: E402

METRIC = "attn fwd TFLOP/s (causal-adj) & % bf16 MFMA peak; decode HBM GB/s"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "exact_attention_08_amd", "csrc")
COPY_BYTES = 1 << 30          # plain-copy calibration: 1 GiB read + 1 GiB written


def source_hash(name: str) -> str:
    """sha256 of a kernel source file and the two headers every kernel file
    includes (ties profiled counters to the code)."""
    h = hashlib.sha256()
    for f in (name, "fa_device.hpp", "fa_internal.hpp"):
        with open(os.path.join(KERNEL_SRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(summary: str, src: str):
    """HBM bytes per launch recorded in a committed rocprofv3 summary, or None
    when the summary is missing or the kernel source changed since."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not t or h.group(1) != source_hash(src):
        return None
    return int(t.group(1))


def copy_calibration():
    """A plain device copy of known size, run under rocprofv3 --pmc to scale
    FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "copies": 3}), flush=True)


# Untimed calls before each leg's W warm-up calls, so that the timed steps
# run at the GPU's sustained clock: from idle the clocks ramp up over the
# first tens of milliseconds of load.  Legs are separated by host work
# (input generation), so every leg settles anew.
CLOCK_SETTLE_S = 0.25


def _timed(fn, steps: int, warmup: int):
    """Clock settling (CLOCK_SETTLE_S of untimed calls), W untimed calls,
    then exactly K timed calls bracketed by synchronize, an event before each
    call and one after the last, all on the launch stream.  Returns (wall ms
    per step, {mean, median, min} event ms per call)."""
    t_end = time.perf_counter() + CLOCK_SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record(stream)
        fn()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    stats = {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": per[len(per) // 2],
             "min": per[0]}
    return wall, stats


def _round_stats(st):
    return {k: round(v, 5) for k, v in st.items()}


def fwd_kernel(sq: int, sk: int, causal: bool, window) -> tuple[str, str]:
    """(kernel name, source file) that fa_fwd / fa_fwd_varlen launch for
    sq rows and sk keys (packed: the host bounds): the rule of the host
    launcher (fwd_use_wide: average keys per row above 2560 -> wide)."""
    wl, wr = window
    if wl >= sk - 1:
        wl = -1
    if wr >= sq - 1:
        wr = -1
    kpr = sk - (min(sq, sk) // 2 if causal else 0)
    if wl >= 0 and (causal or wr >= 0):
        kpr = min(kpr, wl + 1 + (0 if causal else wr))
    if kpr > 2560:
        return "fa_fwd_wide_kernel", "fa_fwd_wide.hip"
    return "fa_fwd_kernel", "fa_fwd.hip"


def _roofline(work, stats, kernel, src, workload, hbm_bound=False):
    """Roofline object of one forward leg: algorithmic FLOP (or bytes) per
    launch over the mean launch time on the launch stream; for an HBM-bound
    leg also the fraction of the roofline time max(F / MFMA peak, B / HBM
    peak)."""
    t = stats["mean"] * 1e-3
    tf = work["flop"] / t / 1e12
    gbs = work["bytes"] / t / 1e9
    traffic = profiled_traffic(f"{kernel}_{workload}.md", src)
    if hbm_bound:
        t_roof = max(work["flop"] / (metrics.PEAK_BF16_TFLOPS * 1e12),
                     work["bytes"] / (metrics.PEAK_HBM_GBS * 1e9))
        return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1),
                "peak": metrics.PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / metrics.PEAK_HBM_GBS, 4),
                "time_at_roofline_ms": round(t_roof * 1e3, 5),
                "frac_of_roofline_time": round(t_roof / t, 4),
                "tflops": round(tf, 2), "frac_bf16_mfma_peak": round(tf / metrics.PEAK_BF16_TFLOPS, 4),
                "avg_launch_ms": round(stats["mean"], 5), "traffic": traffic}
    return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2),
            "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / metrics.PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(stats["mean"], 5), "traffic": traffic}


def bench_fwd_padded(steps, warmup, w, inputs=None):
    """fa_fwd on a padded workload; returns (inputs, work, wall, stats, leg)."""
    q, k, v = inputs if inputs is not None else synth.generate(w)
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    work = metrics.fwd_work(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window)

    def step():
        fa.fwd(qd, kd, vd, causal=w.causal, window=w.window, out=out, lse=lse)

    wall, stats = _timed(step, steps, warmup)
    kernel, src = fwd_kernel(w.Sq, w.Sk, w.causal, w.window)
    hbm = work["flop"] / work["bytes"] < metrics.PEAK_BF16_TFLOPS * 1e12 / (metrics.PEAK_HBM_GBS * 1e9)
    leg = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk,
           "d": w.d, "dtype": w.dtype, "causal": w.causal, "window": list(w.window),
           "algorithmic_flop": work["flop"], "algorithmic_bytes": work["bytes"],
           "ms_per_call": _round_stats(stats), "steps": steps,
           "roofline": _roofline(work, stats, kernel, src, w.name, hbm_bound=hbm)}
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    return (q, k, v), work, wall, stats, leg


def bench_fwd_varlen(steps, warmup, w):
    q, k, v, cu, lens = synth.generate(w)
    dev = "cuda:0"
    qd, kd, vd, cud = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    mx = int(lens.max())
    out = torch.empty_like(qd)
    lse = torch.empty((w.Hq, qd.shape[0]), dtype=torch.float32, device=dev)
    work = metrics.varlen_work(lens.tolist(), lens.tolist(), w.Hq, w.Hkv, w.d, w.causal, w.window)

    def step():
        fa.fwd_varlen(qd, kd, vd, cud, cud, mx, mx, causal=w.causal, window=w.window, out=out,
                      lse=lse)

    wall, stats = _timed(step, steps, warmup)
    kernel, src = fwd_kernel(mx, mx, w.causal, w.window)
    leg = {"workload": w.name, "sequences": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
           "dtype": w.dtype, "causal": w.causal, "total_tokens": int(cu[-1]), "max_len": mx,
           "algorithmic_flop": work["flop"], "algorithmic_bytes": work["bytes"],
           "ms_per_call": _round_stats(stats), "steps": steps,
           "roofline": _roofline(work, stats, kernel, src, w.name)}
    del qd, kd, vd, cud, out, lse
    torch.cuda.empty_cache()
    return leg


def bench_fwd_mod(steps, warmup, w, qd, kd, vd, softcap, alibi):
    """fa_fwd_mod on the prefill workload's resident inputs: ALiBi (the usual
    geometric slopes 2^(-8 (h+1) / Hq)) and/or soft-capping.  FLOP as the
    plain forward (the modifier arithmetic is not counted)."""
    slopes = None
    if alibi:
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.Hq) for h in range(w.Hq)],
                              dtype=torch.float32, device=qd.device)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=qd.device)
    work = metrics.fwd_work(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window)

    def step():
        fa.fwd_mod(qd, kd, vd, causal=w.causal, window=w.window, alibi_slopes=slopes,
                   softcap=softcap, out=out, lse=lse)

    wall, stats = _timed(step, steps, warmup)
    tf = work["flop"] / (stats["mean"] * 1e-3) / 1e12
    name = "+".join(x for x, on in (("alibi", alibi), (f"softcap{softcap:g}", softcap > 0)) if on)
    return {"workload": f"{w.name}_{name}", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_step": round(wall, 4), "ms_per_call": _round_stats(stats),
            "frac_bf16_mfma_peak": round(tf / metrics.PEAK_BF16_TFLOPS, 4)}


def bench_fp8(steps, warmup, w):
    """fa_fwd_fp8 on the prefill workload's shape: fp32 N(0, 1) inputs drawn
    from its seed, quantised per tensor to e4m3 (synth.gen_fp8), resident in
    HBM; two kernels per call (V transpose into the workspace, attention).
    FLOP as the 16-bit forward; peaks: fp8 dense MFMA and bf16 for context."""
    (q8, k8, v8), (dq, dk, dv) = synth.gen_fp8(w.seed, w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.sigma)
    dev = "cuda:0"
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fwd_fp8_workspace_bytes(w.B, w.Hkv, w.Sk, w.d), dtype=torch.uint8, device=dev)
    work = metrics.fwd_work(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window)

    def step():
        fa.fwd_fp8(q8, k8, v8, dq, dk, dv, causal=w.causal, window=w.window, out=out, lse=lse,
                   workspace=ws)

    wall, stats = _timed(step, steps, warmup)
    tf = work["flop"] / (stats["mean"] * 1e-3) / 1e12
    res = {"workload": f"{w.name}_fp8_e4m3", "value": round(tf, 2), "unit": "TFLOP/s",
           "ms_per_step": round(wall, 4), "ms_per_call": _round_stats(stats),
           "frac_fp8_mfma_peak": round(tf / metrics.PEAK_FP8_TFLOPS, 4),
           "frac_bf16_mfma_peak": round(tf / metrics.PEAK_BF16_TFLOPS, 4), "kernels_per_call": 2}
    del q8, k8, v8, out, lse, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(steps, warmup):
    w = synth.WORKLOADS["kvcache_decode"]
    q, kc, vc, sl = synth.generate(w)
    dev = "cuda:0"
    qd, kd, vd, sld = q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev)
    del kc, vc
    mx = int(sl.max())
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.Hq, mx, w.d, w.split), dtype=torch.uint8,
                     device=dev)
    work = metrics.decode_work(sl.tolist(), w.Hq, w.Hkv, w.d)

    def step():
        fa.decode_kvcache(qd, kd, vd, sld, mx, split_size=w.split, out=out, lse=lse, workspace=ws)

    wall, stats = _timed(step, steps, warmup)
    gbs = work["bytes"] / (stats["mean"] * 1e-3) / 1e9
    res = {"workload": w.name, "value": round(gbs, 1), "unit": "GB/s",
           "ms_per_step": round(wall, 4), "ms_per_call": _round_stats(stats),
           "frac_hbm_peak": round(gbs / metrics.PEAK_HBM_GBS, 4),
           "algorithmic_bytes": work["bytes"], "kernels_per_call": 2,
           "cache_lengths": {"min": int(sl.min()), "max": mx, "sum": int(sl.sum())}}
    del qd, kd, vd
    torch.cuda.empty_cache()
    return res


def bench_decode_paged(steps, warmup, page_size=256):
    """fa_decode_paged on the decode workload's keys and values: the same
    drawn lengths and rows cut into pages of page_size rows placed in a
    shuffled pool; each sequence's last key arrives as the appended new
    token (written into its page by the call, then attended), so the
    attended keys, and the algorithmic bytes, are those of the contiguous
    decode."""
    w = synth.WORKLOADS["kvcache_decode"]
    q, kp, vp, bt, sl, kn, vn, lens = synth.gen_paged(
        w.seed, w.B, w.Hq, w.Hkv, w.d, page_size, w.len_range[0], w.len_range[1], w.dtype,
        w.sigma, append=True)
    dev = "cuda:0"
    qd, kpd, vpd, btd, sld, knd, vnd = (x.to(dev) for x in (q, kp, vp, bt, sl, kn, vn))
    del kp, vp
    mx = int(lens.max())
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.Hq, mx, w.d, w.split), dtype=torch.uint8,
                     device=dev)
    work = metrics.decode_work(lens.tolist(), w.Hq, w.Hkv, w.d)

    def step():
        fa.decode_paged(qd, kpd, vpd, btd, sld, mx, k_new=knd, v_new=vnd, split_size=w.split,
                        out=out, lse=lse, workspace=ws)

    wall, stats = _timed(step, steps, warmup)
    gbs = work["bytes"] / (stats["mean"] * 1e-3) / 1e9
    res = {"workload": w.name + f"_paged{page_size}_append", "value": round(gbs, 1), "unit": "GB/s",
           "ms_per_step": round(wall, 4), "ms_per_call": _round_stats(stats),
           "frac_hbm_peak": round(gbs / metrics.PEAK_HBM_GBS, 4),
           "algorithmic_bytes": work["bytes"], "kernels_per_call": 3,
           "page_size": page_size, "num_pages": int(kpd.shape[0])}
    del qd, kpd, vpd, btd, sld, knd, vnd
    torch.cuda.empty_cache()
    return res


def bench_backward(steps, warmup, w):
    """fa_bwd (two kernels) on the same workload, with the GPU forward's own
    O and LSE and a seeded incoming gradient, all resident in HBM."""
    q, k, v = synth.generate(w)
    dev = "cuda:0"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    god = synth.gen_grad(w.seed + 1000, qd.shape, w.dtype).to(dev)
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, window=w.window)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(max(fa.bwd_workspace_bytes(w.B, w.Hq, w.Sq), 16), dtype=torch.uint8, device=dev)
    work = metrics.bwd_work(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window)

    def step():
        fa.bwd(qd, kd, vd, o, god, lse, causal=w.causal, window=w.window, dq=dq, dk=dk, dv=dv,
               workspace=ws)

    wall, stats = _timed(step, steps, warmup)
    tf = work["flop"] / (stats["mean"] * 1e-3) / 1e12
    res = {"workload": w.name, "value": round(tf, 2), "unit": "TFLOP/s",
           "ms_per_step": round(wall, 4), "ms_per_call": _round_stats(stats),
           "frac_bf16_mfma_peak": round(tf / metrics.PEAK_BF16_TFLOPS, 4),
           "algorithmic_flop": work["flop"], "kernels_per_call": 2,
           "flop_convention": "10*d per visible pair per query head (2.5x forward)"}
    del qd, kd, vd, god, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(q, k, v, w, budget_s: float):
    """The fp64 oracle on the host cores, as it stands (not tuned for this):
      * all threads over whole (sequence, head) slices of the headline
        workload, as many as fit in about budget_s seconds (the line's value);
      * one thread on the whole small non-causal workload;
      * one thread on a sample of the KV-cache decode workload (4 sequences
        with lengths drawn like the workload's), as GB/s of the visible cache
        bytes it reads."""
    import oracle
    orc = oracle.Oracle()
    threads = orc.set_threads(0)
    G = w.Hq // w.Hkv
    n_done, flop, t_total = 0, 0, 0.0
    rows = list(range(w.Sq))
    for b in range(w.B):
        for h in range(w.Hq):
            t0 = time.perf_counter()
            orc.attention_rows(q[b, :, h], rows, w.Sq, k[b, :, h // G], v[b, :, h // G],
                               causal=w.causal, window=w.window, scale=w.scale)
            t_total += time.perf_counter() - t0
            n_done += 1
            flop += 4 * w.d * metrics.visible_pairs(w.Sq, w.Sk, w.causal, w.window)
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    res = {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n_done} of {w.B * w.Hq} (sequence, head) slices of {w.name}, all "
                     f"{w.Sq} rows each, fp64, {t_total:.1f} s on {threads} threads"}
    orc.set_threads(1)
    try:
        ws = synth.WORKLOADS["small_noncausal"]
        q1, k1, v1 = synth.generate(ws)
        t0 = time.perf_counter()
        orc.attention(q1, k1, v1, causal=ws.causal, window=ws.window, scale=ws.scale)
        t1 = time.perf_counter() - t0
        f1 = metrics.fwd_work(ws.B, ws.Hq, ws.Hkv, ws.Sq, ws.Sk, ws.d, ws.causal, ws.window)
        wd = synth.WORKLOADS["kvcache_decode"]
        lens = synth.gen_lengths(torch.Generator().manual_seed(wd.seed), 4, *wd.len_range)
        qd, kc, vc, sl = synth.gen_decode(wd.seed, 4, wd.Hq, wd.Hkv, wd.d, int(lens.max()), 0, 0,
                                          wd.dtype, lengths=lens.tolist())
        t0 = time.perf_counter()
        orc.attention_decode(qd, kc, vc, sl, causal=True, scale=wd.scale)
        t5 = time.perf_counter() - t0
        d5 = metrics.decode_work(sl.tolist(), wd.Hq, wd.Hkv, wd.d)
        res["single_thread"] = {
            "small_noncausal": {"value": round(f1["flop"] / t1 / 1e9, 3), "unit": "GFLOP/s",
                                "seconds": round(t1, 4), "sample": "the whole workload"},
            "kvcache_decode": {"value": round(d5["bytes"] / t5 / 1e9, 3), "unit": "GB/s",
                               "gflops": round(d5["flop"] / t5 / 1e9, 3), "seconds": round(t5, 3),
                               "sample": f"4 sequences, cache lengths {sl.tolist()}"}}
    finally:
        orc.set_threads(threads)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="causal_gqa_prefill",
                    choices=[n for n, w in synth.WORKLOADS.items() if w.kind == "fwd"])
    ap.add_argument("--no-configs", action="store_true", help="skip the other forward workloads")
    ap.add_argument("--only-config", default=None,
                    help="time only this forward workload (with --no-* flags: profiling)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-mods", action="store_true", help="skip the score-modifier legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit forward leg")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this attention build runs on exactly one GPU; --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    fa.load()   # fails loudly if the HIP library is not built

    if args.only_config is not None:
        w = synth.WORKLOADS[args.only_config]
        if w.kind == "varlen":
            leg = bench_fwd_varlen(args.steps, args.warmup, w)
        else:
            leg = bench_fwd_padded(args.steps, args.warmup, w)[4]
        print(json.dumps(leg), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    (q, k, v), work, wall, stats, leg = bench_fwd_padded(args.steps, args.warmup, w)
    tflops_wall = work["flop"] / (wall * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tflops_wall, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": CLOCK_SETTLE_S,
        "ms_per_step": round(wall, 5),
        "ms_per_call": leg["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Sk": w.Sk, "d": w.d, "causal": w.causal, "window": list(w.window),
                   "algorithmic_flop": work["flop"], "algorithmic_bytes": work["bytes"],
                   "frac_bf16_mfma_peak": round(tflops_wall / metrics.PEAK_BF16_TFLOPS, 4)},
        "roofline": leg["roofline"],
    }
    if not args.no_mods:
        qd, kd, vd = q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0")
        ms, mw = max(5, args.steps // 4), max(2, args.warmup // 4)
        line["forward_modifiers"] = [bench_fwd_mod(ms, mw, w, qd, kd, vd, 0.0, True),
                                     bench_fwd_mod(ms, mw, w, qd, kd, vd, 50.0, False),
                                     bench_fwd_mod(ms, mw, w, qd, kd, vd, 50.0, True)]
        del qd, kd, vd
        torch.cuda.empty_cache()
    if not args.no_configs:
        cs, cw = max(10, args.steps // 2), max(3, args.warmup // 2)
        legs = {}
        for name in ("small_noncausal", "causal_window", "varlen_causal", "long_causal_prefill"):
            if name == w.name:
                continue
            wx = synth.WORKLOADS[name]
            if wx.kind == "varlen":
                legs[name] = bench_fwd_varlen(cs, cw, wx)
            elif name == "long_causal_prefill":
                legs[name] = bench_fwd_padded(max(5, args.steps // 5), max(2, args.warmup // 5), wx)[4]
            else:
                legs[name] = bench_fwd_padded(cs, cw, wx)[4]
        line["configs"] = legs
    if not args.no_fp8:
        line["forward_fp8"] = bench_fp8(max(10, args.steps // 2), max(3, args.warmup // 2), w)
    if not args.no_decode:
        line["decode"] = bench_decode(max(10, args.steps // 2), max(3, args.warmup // 2))
        line["decode_paged"] = bench_decode_paged(max(10, args.steps // 2), max(3, args.warmup // 2))
    if not args.no_backward:
        line["backward"] = bench_backward(max(5, args.steps // 5), max(2, args.warmup // 5), w)
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(q, k, v, w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
