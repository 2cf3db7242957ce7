"""GPU parity: the HIP path through the C ABI against the fp64 oracle,
element by element, on seeded inputs that span several tiles with ragged
tails, plus the degenerate cases (empty key sets, single key, single query,
fully masked rows, zero and negative scale).

Tolerance: max |dO| <= 1e-2, max |dLSE| <= 1e-3 against the unrounded fp64
oracle (see oracle/checks.py for the one-ulp rule on |O| >= 2)."""
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth
from oracle.checks import compare, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, B, Hq, Hkv, Sq, Sk, d, dtype, causal, window, scale, seed
FWD_CASES = [
    ("small_noncausal_full", 1, 1, 1, 256, 256, 64, "bf16", False, (-1, -1), None, 1),
    ("causal_gqa_ragged", 2, 8, 2, 300, 300, 128, "bf16", True, (-1, -1), None, 101),
    ("noncausal_mha_fp16", 1, 4, 4, 200, 333, 128, "fp16", False, (-1, -1), None, 102),
    ("noncausal_d64_ragged", 2, 4, 1, 130, 257, 64, "bf16", False, (-1, -1), None, 103),
    ("causal_d64_fp16", 1, 6, 3, 384, 384, 64, "fp16", True, (-1, -1), None, 104),
    ("causal_sq_lt_sk", 1, 4, 2, 77, 300, 128, "bf16", True, (-1, -1), None, 105),
    ("causal_sq_gt_sk", 1, 4, 2, 300, 77, 128, "bf16", True, (-1, -1), None, 106),
    ("window_causal", 1, 4, 4, 700, 700, 128, "fp16", True, (100, 100), None, 107),
    ("window_two_sided", 1, 2, 1, 400, 400, 128, "bf16", False, (50, 30), None, 108),
    ("window_zero", 1, 2, 2, 200, 200, 64, "bf16", True, (0, 0), None, 109),
    ("window_left_only", 1, 2, 2, 260, 260, 128, "bf16", False, (70, -1), None, 110),
    ("window_right_only", 1, 2, 2, 260, 300, 128, "fp16", False, (-1, 40), None, 111),
    ("window_d64_causal", 2, 4, 2, 500, 500, 64, "bf16", True, (130, -1), None, 112),
    # sliding windows: also with Sq != Sk (the bottom-right alignment
    # shifts the band) and a wide band over four query heads per work-group
    ("window_sq_lt_sk", 1, 4, 2, 150, 420, 128, "bf16", True, (64, -1), None, 113),
    ("window_sq_gt_sk_d64", 1, 4, 2, 420, 150, 64, "fp16", False, (40, 20), None, 114),
    ("window_gqa_wide", 1, 8, 2, 600, 600, 128, "bf16", True, (300, -1), None, 115),
    ("negative_scale", 1, 2, 2, 150, 150, 128, "bf16", True, (-1, -1), -0.09, 113),
    ("zero_scale", 1, 2, 2, 150, 150, 128, "bf16", False, (-1, -1), 0.0, 114),
    ("single_query", 2, 8, 2, 1, 500, 128, "bf16", True, (-1, -1), None, 115),
    ("single_key", 1, 2, 2, 50, 1, 128, "bf16", False, (-1, -1), None, 116),
    ("empty_keys", 1, 2, 2, 40, 0, 128, "bf16", False, (-1, -1), None, 117),
    ("large_group", 1, 16, 1, 130, 130, 128, "bf16", True, (-1, -1), None, 118),
    ("xcd_grouped_heads", 2, 16, 4, 256, 256, 128, "bf16", True, (-1, -1), None, 119),
    ("xcd_grouped_d64", 4, 8, 2, 200, 200, 64, "fp16", True, (-1, -1), None, 120),
    ("sigma_large_scores", 1, 4, 2, 256, 256, 128, "bf16", True, (-1, -1), 0.5, 121),
    # rows of 2,000-3,000 keys on the paired kernel (32-row waves)
    ("long_causal_sq_lt_sk", 1, 4, 2, 300, 2500, 128, "bf16", True, (-1, -1), None, 131),
    ("long_noncausal_ragged", 1, 2, 1, 200, 2113, 128, "fp16", False, (-1, -1), None, 132),
    ("long_causal_gqa", 1, 8, 2, 2200, 2200, 128, "bf16", True, (-1, -1), None, 133),
    ("long_d64_fp16", 2, 4, 2, 150, 2090, 64, "fp16", True, (-1, -1), None, 134),
    ("long_window_left", 1, 4, 4, 2400, 2400, 128, "bf16", True, (2100, -1), None, 135),
    ("long_window_two_sided", 1, 2, 2, 100, 3000, 128, "bf16", False, (1500, 1000), None, 136),
    ("long_causal_sq_gt_sk", 1, 2, 2, 2300, 2100, 128, "bf16", True, (-1, -1), None, 137),
    ("long_negative_scale", 1, 2, 1, 64, 2049, 64, "bf16", False, (-1, -1), -0.07, 138),
    ("long_group3", 1, 6, 2, 128, 2300, 128, "bf16", True, (-1, -1), None, 139),
    # rows that see more than 2,560 keys on average run on the wide kernel
    # (64-row waves): the same mask modes and edge cases on that side
    ("wide_causal_sq_lt_sk", 1, 4, 2, 300, 3000, 128, "bf16", True, (-1, -1), None, 141),
    ("wide_noncausal_ragged", 1, 2, 1, 200, 2613, 128, "fp16", False, (-1, -1), None, 142),
    ("wide_causal_gqa", 1, 8, 2, 5200, 5200, 128, "bf16", True, (-1, -1), None, 143),
    ("wide_d64_fp16", 2, 4, 2, 150, 2700, 64, "fp16", True, (-1, -1), None, 144),
    ("wide_window_left", 1, 4, 4, 5400, 5400, 128, "bf16", True, (2600, -1), None, 145),
    ("wide_window_two_sided", 1, 2, 2, 100, 3000, 128, "bf16", False, (1500, 1100), None, 146),
    ("wide_causal_sq_gt_sk", 1, 2, 2, 6000, 5300, 128, "bf16", True, (-1, -1), None, 147),
    ("wide_negative_scale", 1, 2, 1, 64, 2600, 64, "bf16", False, (-1, -1), -0.07, 148),
    ("wide_group3", 1, 6, 2, 128, 2800, 128, "bf16", True, (-1, -1), None, 149),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_matches_oracle(case):
    name, B, Hq, Hkv, Sq, Sk, d, dt, causal, window, scale, seed = case
    q, k, v = synth.gen_padded(seed, B, Hq, Hkv, Sq, Sk, d, dt)
    print(f"[case] fwd {case}", flush=True)
    o, lse = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window,
                    softmax_scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal=causal, window=window, scale=scale)
    log(compare(o, lse, ro, rl, dt, name), name)


# name, lengths_q, lengths_k (None = same), Hq, Hkv, d, dtype, causal, window, seed
VARLEN_CASES = [
    ("ragged_causal", [1, 127, 128, 129, 300, 0, 64, 2], None, 8, 2, 128, "bf16", True,
     (-1, -1), 201),
    ("separate_lengths", [5, 200, 0, 33], [7, 150, 3, 0], 4, 4, 128, "bf16", False,
     (-1, -1), 202),
    ("window_d64_fp16", [90, 257, 31], None, 4, 1, 64, "fp16", True, (32, 0), 203),
    ("many_short_xcd", [40, 7, 130, 66, 1, 99, 128, 255], None, 8, 1, 128, "bf16", True,
     (-1, -1), 204),
    # longer sequences: the paired kernel up to 2,560 keys per row on
    # average, the wide kernel's packed form beyond
    ("long_packed", [2200, 30, 0, 700], None, 4, 2, 128, "bf16", True, (-1, -1), 205),
    ("long_packed_d64", [100, 2100], [2300, 2100], 2, 2, 64, "fp16", False, (-1, -1), 206),
    ("wide_packed", [5400, 30, 0, 700], None, 4, 2, 128, "bf16", True, (-1, -1), 207),
    ("wide_packed_d64", [100, 2100], [2700, 2100], 2, 2, 64, "fp16", False, (-1, -1), 208),
    # the longest-first order of up to 64 packed sequences: K/V heads that
    # straddle XCDs (16) or share one (2), key lengths that differ from the
    # query lengths, empty sequences, and more sequences than the order sorts
    ("sorted_hkv16", [300, 0, 1000, 64, 65, 2], [40, 700, 1000, 64, 300, 2], 32, 16, 128, "bf16",
     True, (-1, -1), 209),
    ("sorted_hkv2", [33, 700, 5, 0, 128, 129, 900, 31, 64, 1, 250, 400], None, 8, 2, 128, "bf16",
     True, (-1, -1), 210),
    ("sorted_64_seqs", [(37 * i) % 260 for i in range(64)], None, 8, 1, 128, "bf16", True,
     (-1, -1), 211),
    ("unsorted_72_seqs", [(53 * i) % 190 for i in range(72)], None, 8, 1, 64, "fp16", True,
     (-1, -1), 212),
    ("sorted_wide", [5400, 30, 0, 7000, 2000, 6000, 1, 100], None, 4, 1, 128, "bf16", True,
     (-1, -1), 213),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_matches_oracle(case):
    name, lq, lk, Hq, Hkv, d, dt, causal, window, seed = case
    lk = lq if lk is None else lk
    gen = torch.Generator().manual_seed(seed)
    t = synth.DTYPES[dt]
    q = torch.randn(sum(lq), Hq, d, generator=gen).to(t)
    k = torch.randn(sum(lk), Hkv, d, generator=gen).to(t)
    v = torch.randn(sum(lk), Hkv, d, generator=gen).to(t)
    cq, ck = synth.cumulative(lq), synth.cumulative(lk)
    print(f"[case] varlen {case}", flush=True)
    o, lse = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), max(lq),
                           max(lk), causal=causal, window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(q, k, v, cq, ck, causal=causal, window=window,
                                     scale=d ** -0.5)
    log(compare(o, lse, ro, rl, dt, name), name)


# name, B, Hq, Hkv, cap, lens, d, dtype, causal, window, split, seed
DECODE_CASES = [
    ("gqa_split1024", 4, 8, 2, 2560, [1, 63, 1024, 2500], 128, "bf16", True, (-1, -1), 1024, 301),
    ("gqa_split64", 4, 8, 2, 2560, [1, 63, 1024, 2500], 128, "bf16", False, (-1, -1), 64, 302),
    ("mha_split256", 3, 4, 4, 1000, [1000, 500, 33], 128, "fp16", True, (-1, -1), 256, 303),
    ("group40_two_qblocks", 2, 40, 1, 700, [700, 129], 128, "bf16", True, (-1, -1), 128, 304),
    ("window_left", 3, 8, 2, 3000, [3000, 100, 1500], 128, "bf16", True, (200, -1), 512, 305),
    ("d64_fp16", 3, 16, 4, 1200, [1200, 1, 640], 64, "fp16", True, (-1, -1), 256, 306),
    ("empty_cache_row", 2, 4, 1, 300, [0, 300], 128, "bf16", True, (-1, -1), 128, 307),
    ("split192_window", 2, 8, 2, 2000, [1999, 700], 128, "bf16", True, (300, -1), 192, 308),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_oracle(case):
    name, B, Hq, Hkv, cap, lens, d, dt, causal, window, split, seed = case
    q, kc, vc, sl = synth.gen_decode(seed, B, Hq, Hkv, d, cap, 0, 0, dt, lengths=lens)
    print(f"[case] decode {case}", flush=True)
    o, lse = fa.decode_kvcache(q.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV), max(max(lens), 1),
                               causal=causal, window=window, split_size=split)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_decode(q, kc, vc, sl, causal=causal, window=window, scale=d ** -0.5)
    log(compare(o, lse, ro, rl, dt, name), name)


def test_lse_may_be_omitted():
    q, k, v = synth.gen_padded(401, 1, 4, 2, 200, 200, 128, "bf16")
    print("[case] fwd without lse", flush=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, _ = fa.fwd(qd, kd, vd, causal=True)
    out = torch.empty_like(qd)
    st = fa.load().fa_fwd(fa._ptr(qd), fa._ptr(kd), fa._ptr(vd), fa._ptr(out), None, 1, 4, 2, 200,
                          200, 128, 1, -1, -1, 128 ** -0.5, 0, fa._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, out)
