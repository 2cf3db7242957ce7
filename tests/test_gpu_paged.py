"""GPU parity of the paged-cache decode (fa_decode_paged through the C ABI)
against the fp64 oracle, with and without appending the new token: outputs
and LSE within the forward's tolerance, the page pools after the call
bitwise equal to the oracle's (exactly one row per sequence and K/V head
written), and invariants that hold bitwise because the paged and contiguous
paths share the split arithmetic: a paged cache gives the contiguous
decode's bits, garbage in unreferenced rows and pages has no effect, and a
second call that reads the appended rows from the cache reproduces the
first."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth
from oracle.checks import compare, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, B, Hq, Hkv, d, dtype, page_size, lengths (keys attended), append, window, split, seed
PAGED_CASES = [
    ("page32_append_gqa", 5, 8, 2, 128, "bf16", 32, [1, 31, 32, 33, 700], True, (-1, -1), 64, 501),
    ("page256_no_append", 3, 32, 8, 128, "bf16", 256, [1, 256, 2000], False, (-1, -1), 1024, 502),
    ("page64_d64_fp16_window", 4, 4, 4, 64, "fp16", 64, [5, 64, 65, 1000], True, (100, -1), 128,
     503),
    ("page1024_group16", 2, 16, 1, 128, "bf16", 1024, [3000, 1], True, (-1, -1), 1024, 504),
    ("page32_mha_many_splits", 2, 8, 8, 128, "bf16", 32, [4096, 2049], False, (-1, -1), 256, 505),
    ("page96_split192", 3, 8, 2, 128, "bf16", 96, [97, 1, 1500], True, (300, -1), 192, 506),
]


def _inputs(case):
    name, B, Hq, Hkv, d, dt, ps, lens, append, window, split, seed = case
    return synth.gen_paged(seed, B, Hq, Hkv, d, ps, 0, 0, dt, lengths=lens, append=append,
                           spare_pages=3)


def _run(q, kp, vp, bt, sl, kn, vn, max_len, window, split):
    o, lse = fa.decode_paged(q, kp, vp, bt, sl, max_len, k_new=kn, v_new=vn, causal=True,
                             window=window, split_size=split)
    torch.cuda.synchronize()
    return o, lse


def _dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_matches_oracle(case):
    name, B, Hq, Hkv, d, dt, ps, lens, append, window, split, seed = case
    print(f"[case] paged {case}", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = _inputs(case)
    qd, kpd, vpd, btd, sld, knd, vnd = _dev(q, kp, vp, bt, sl, kn, vn)
    o, lse = _run(qd, kpd, vpd, btd, sld, knd, vnd, max(lens), window, split)
    ro, rl, rkp, rvp = oracle.attention_decode_paged(q, kp, vp, bt, sl, kn, vn, causal=True,
                                                     window=window, scale=d ** -0.5)
    log(compare(o, lse, ro, rl, dt, name), name)
    t = synth.DTYPES[dt]
    assert torch.equal(kpd.cpu(), torch.from_numpy(rkp).to(t)), f"{name}: k pages differ"
    assert torch.equal(vpd.cpu(), torch.from_numpy(rvp).to(t)), f"{name}: v pages differ"
    changed = (kpd.cpu() != kp).any(-1).any(-1).sum().item()
    assert changed <= (B if append else 0), f"{name}: {changed} page rows changed"


@pytest.mark.parametrize("case", PAGED_CASES[:4], ids=[c[0] for c in PAGED_CASES[:4]])
def test_paged_equals_contiguous_bitwise(case):
    """Same seed, same keys: the paged call (with or without append) gives
    the contiguous-cache decode's exact bits."""
    name, B, Hq, Hkv, d, dt, ps, lens, append, window, split, seed = case
    print(f"[case] paged vs contiguous {name}", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = _inputs(case)
    o, lse = _run(*_dev(q, kp, vp, bt, sl, kn, vn), max(lens), window, split)
    q2, kc, vc, sl2 = synth.gen_decode(seed, B, Hq, Hkv, d, max(lens), 0, 0, dt, lengths=lens)
    assert torch.equal(q, q2)
    o2, lse2 = fa.decode_kvcache(q2.to(DEV), kc.to(DEV), vc.to(DEV), sl2.to(DEV), max(lens),
                                 causal=True, window=window, split_size=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_paged_garbage_has_no_effect():
    """Finite garbage (+-1e4) in page rows past each sequence's keys and in
    unreferenced pages leaves the bits unchanged."""
    case = PAGED_CASES[0]
    name, B, Hq, Hkv, d, dt, ps, lens, append, window, split, seed = case
    print("[case] paged garbage", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = _inputs(case)
    o1, l1 = _run(*_dev(q, kp, vp, bt, sl, kn, vn), max(lens), window, split)
    used = torch.zeros(kp.shape[:2], dtype=torch.bool)
    for b in range(B):
        for t in range(int(L[b])):
            used[int(bt[b, t // ps]), t % ps] = True
    gen = torch.Generator().manual_seed(77)
    for pool in (kp, vp):
        g = (torch.randint(0, 2, pool.shape, generator=gen) * 2 - 1).to(pool.dtype) * 1e4
        pool[~used] = g[~used]
    o2, l2 = _run(*_dev(q, kp, vp, bt, sl, kn, vn), max(lens), window, split)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_second_call_reads_appended_rows():
    """After an append, a call without one over cache_seqlens + 1 keys reads
    the appended rows from the pages and reproduces the first result."""
    case = PAGED_CASES[2]
    name, B, Hq, Hkv, d, dt, ps, lens, append, window, split, seed = case
    print("[case] paged append then read", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = _inputs(case)
    qd, kpd, vpd, btd, sld, knd, vnd = _dev(q, kp, vp, bt, sl, kn, vn)
    o1, l1 = _run(qd, kpd, vpd, btd, sld, knd, vnd, max(lens), window, split)
    o2, l2 = _run(qd, kpd, vpd, btd, sld + 1, None, None, max(lens), window, split)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_length_clamped_to_bound():
    """Cache lengths beyond the host bound are clamped on the device (with
    an append: the new row goes to position max_seqlen_k - 1)."""
    print("[case] paged clamp", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = synth.gen_paged(508, 2, 4, 2, 128, 64, 0, 0, "bf16",
                                                   lengths=[128, 70], append=True)
    bound = 100
    sl_big = torch.tensor([500, 69], dtype=torch.int32)      # 500 > bound - 1: clamped to 99
    qd, kpd, vpd, btd, sld, knd, vnd = _dev(q, kp, vp, bt, sl_big, kn, vn)
    o, lse = _run(qd, kpd, vpd, btd, sld, knd, vnd, bound, (-1, -1), 64)
    ro, rl, rkp, _ = oracle.attention_decode_paged(q, kp, vp, bt, torch.tensor([99, 69]), kn, vn,
                                                   causal=True, scale=128 ** -0.5)
    log(compare(o, lse, ro, rl, "bf16", "paged_clamp"), "paged_clamp")
    assert torch.equal(kpd.cpu(), torch.from_numpy(rkp).to(torch.bfloat16))


def test_paged_empty_cache_with_append_sees_only_new_token():
    """cache_seqlens = 0 with an append: the only key is the new one, so O is
    its value row (to output rounding) and LSE = scale * q . k_new."""
    print("[case] paged empty + append", flush=True)
    q, kp, vp, bt, sl, kn, vn, L = synth.gen_paged(509, 3, 8, 2, 128, 32, 0, 0, "bf16",
                                                   lengths=[1, 1, 1], append=True)
    o, lse = _run(*_dev(q, kp, vp, bt, sl, kn, vn), 1, (-1, -1), 64)
    G = 4
    for b in range(3):
        for h in range(8):
            assert torch.equal(o[b, 0, h].cpu(), vn[b, 0, h // G])
            s = float((q[b, 0, h].double() * kn[b, 0, h // G].double()).sum()) * 128 ** -0.5
            assert abs(lse[b, h].item() - s) < 1e-3
    assert np.isfinite(lse.cpu().numpy()).all()
