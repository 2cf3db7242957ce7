"""GPU parity of the forward with score modifiers (fa_fwd_mod through the C
ABI: ALiBi bias -slope_h * |pos_i - j| and soft-capping cap * tanh(s / cap))
against the fp64 oracle, element by element, with the forward's tolerance
(max |dO| <= 1e-2, max |dLSE| <= 1e-3), on inputs spanning several tiles
with ragged tails and every mask mode; zero slopes reproduce the plain
forward's bits."""
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth
from oracle.checks import compare, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def alibi_slopes(H):
    """The usual geometric slopes 2^(-8 (h+1) / H)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


# name, B, Hq, Hkv, Sq, Sk, d, dtype, causal, window, scale, softcap, alibi, sigma, seed
MOD_CASES = [
    ("alibi_causal_gqa", 2, 8, 2, 300, 300, 128, "bf16", True, (-1, -1), None, 0.0, True, 1.0, 601),
    ("alibi_noncausal_sq_ne_sk", 1, 4, 1, 130, 257, 64, "bf16", False, (-1, -1), None, 0.0, True,
     1.0, 602),
    ("softcap30_large_scores", 1, 4, 2, 256, 256, 128, "fp16", True, (-1, -1), 0.5, 30.0, False,
     1.0, 603),
    ("softcap1_strong", 1, 4, 4, 200, 333, 128, "bf16", False, (-1, -1), None, 1.0, False, 1.0, 604),
    ("both_window_causal", 1, 4, 4, 400, 400, 128, "bf16", True, (100, 100), None, 20.0, True, 1.0,
     605),
    ("alibi_window_two_sided", 1, 2, 1, 300, 300, 128, "bf16", False, (50, 30), None, 0.0, True,
     1.0, 606),
    ("softcap_negative_scale", 1, 2, 2, 150, 150, 128, "bf16", True, (-1, -1), -0.2, 10.0, False,
     1.0, 607),
    ("both_d64_fp16_long", 1, 4, 2, 1000, 1000, 64, "fp16", True, (-1, -1), None, 50.0, True, 0.5,
     608),
    ("alibi_group3_d64_fp16", 1, 6, 2, 300, 300, 64, "fp16", True, (-1, -1), None, 0.0, True, 1.0,
     611),
    ("softcap5_group16", 1, 16, 1, 130, 130, 128, "bf16", True, (-1, -1), 0.3, 5.0, False, 1.0, 612),
    ("alibi_sq_gt_sk", 1, 4, 2, 300, 77, 128, "bf16", True, (-1, -1), None, 0.0, True, 1.0, 613),
    # rows that see more than 2560 keys on average: the wide kernel's
    # modifier variants (the cases above run on the paired kernel)
    ("wide_alibi_causal", 1, 4, 2, 5300, 5300, 128, "bf16", True, (-1, -1), None, 0.0, True, 1.0,
     614),
    ("wide_softcap_noncausal", 1, 2, 1, 100, 2700, 128, "bf16", False, (-1, -1), None, 30.0, False,
     1.0, 615),
    ("wide_both_d64_fp16", 1, 2, 2, 200, 3000, 64, "fp16", False, (-1, -1), None, 20.0, True, 1.0,
     616),
]


@pytest.mark.parametrize("case", MOD_CASES, ids=[c[0] for c in MOD_CASES])
def test_mod_matches_oracle(case):
    (name, B, Hq, Hkv, Sq, Sk, d, dt, causal, window, scale, cap, alibi, sigma, seed) = case
    print(f"[case] fwd_mod {case}", flush=True)
    q, k, v = synth.gen_padded(seed, B, Hq, Hkv, Sq, Sk, d, dt, sigma)
    slopes = alibi_slopes(Hq) if alibi else None
    o, lse = fa.fwd_mod(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window,
                        softmax_scale=scale, softcap=cap,
                        alibi_slopes=slopes.to(DEV) if slopes is not None else None)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_mod(q, k, v, causal=causal, window=window, scale=scale, softcap=cap,
                                  alibi_slopes=slopes.double().numpy() if alibi else None)
    log(compare(o, lse, ro, rl, dt, name), name)


@pytest.mark.parametrize("shape", [(2, 8, 2, 300, 300), (1, 4, 2, 5300, 5300)],
                         ids=["paired", "wide"])
def test_zero_slopes_give_the_plain_result(shape):
    """ALiBi with all-zero slopes adds exact zeros and keeps the plain order
    of running maxima (the max initialisation is skipped), so on either
    kernel the modifier path gives the plain forward's bits."""
    B, Hq, Hkv, Sq, Sk = shape
    print(f"[case] fwd_mod zero slopes {shape}", flush=True)
    q, k, v = synth.gen_padded(609, B, Hq, Hkv, Sq, Sk, 128, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.fwd(qd, kd, vd, causal=True)
    o2, l2 = fa.fwd_mod(qd, kd, vd, causal=True, alibi_slopes=torch.zeros(Hq, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_modifier_is_the_plain_forward():
    print("[case] fwd_mod without modifiers", flush=True)
    q, k, v = synth.gen_padded(610, 1, 4, 2, 200, 200, 64, "fp16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.fwd(qd, kd, vd, causal=True, window=(30, -1))
    o2, l2 = fa.fwd_mod(qd, kd, vd, causal=True, window=(30, -1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [
    (2, 8, 2, 700, 700, 128, "bf16", True, (100, 0)),
    (1, 4, 4, 530, 610, 64, "fp16", False, (90, 40)),
], ids=["causal_gqa_d128", "two_sided_sq_lt_sk_d64"])
def test_zero_slope_window_is_the_plain_forward(shape):
    """Sliding windows (the paired kernel, key tiles in rotated order): the
    modifier path with zero ALiBi slopes gives the plain forward's bits."""
    B, Hq, Hkv, Sq, Sk, d, dt, causal, window = shape
    print(f"[case] zero-slope window {shape}", flush=True)
    q, k, v = synth.gen_padded(620, B, Hq, Hkv, Sq, Sk, d, dt)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.fwd(qd, kd, vd, causal=causal, window=window)
    o2, l2 = fa.fwd_mod(qd, kd, vd, causal=causal, window=window,
                        alibi_slopes=torch.zeros(Hq, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
