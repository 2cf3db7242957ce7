"""GPU parity of the backward (fa_bwd through the C ABI) against the fp64
oracle's gradients, element by element, on seeded inputs spanning several
tiles with ragged tails, every mask mode, GQA, and the degenerate cases
(rows that see no key, a single key, no keys, no queries).

The GPU backward takes the GPU forward's own O and LSE, as a training step
would; the oracle differentiates the exact definition.  Tolerance per element
(``error_bounds``): 2^-8 times the sum of the absolute terms of the
element's sum (16-bit P and dS operands), plus the effect of forming the row
term D from the 16-bit forward output, plus 2^-8 |g| (output rounding)."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth
from oracle.checks import check_grad as check
from oracle.checks import grad_error_bounds as error_bounds

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, B, Hq, Hkv, Sq, Sk, d, dtype, causal, window, scale, seed
BWD_CASES = [
    ("causal_gqa_ragged", 2, 8, 2, 300, 300, 128, "bf16", True, (-1, -1), None, 201),
    ("noncausal_mha_fp16", 1, 4, 4, 200, 333, 128, "fp16", False, (-1, -1), None, 202),
    ("noncausal_d64_ragged", 2, 4, 1, 130, 257, 64, "bf16", False, (-1, -1), None, 203),
    ("causal_d64_fp16", 1, 6, 3, 384, 384, 64, "fp16", True, (-1, -1), None, 204),
    ("causal_sq_lt_sk", 1, 4, 2, 77, 300, 128, "bf16", True, (-1, -1), None, 205),
    ("causal_sq_gt_sk", 1, 4, 2, 300, 77, 128, "bf16", True, (-1, -1), None, 206),
    ("window_causal", 1, 4, 4, 400, 400, 128, "fp16", True, (100, 100), None, 207),
    ("window_two_sided", 1, 2, 1, 300, 300, 64, "bf16", False, (50, 30), None, 208),
    ("window_right_only", 1, 2, 2, 260, 300, 128, "bf16", False, (-1, 40), None, 209),
    ("negative_scale", 1, 2, 2, 150, 150, 128, "bf16", True, (-1, -1), -0.09, 210),
    ("single_key", 1, 2, 2, 50, 1, 128, "bf16", False, (-1, -1), None, 211),
    ("single_query", 2, 8, 2, 1, 300, 128, "bf16", True, (-1, -1), None, 212),
    ("large_group", 1, 16, 1, 130, 130, 128, "bf16", True, (-1, -1), None, 213),
    ("sigma_large_scores", 1, 4, 2, 256, 256, 128, "bf16", True, (-1, -1), 0.5, 214),
    ("long_causal", 1, 4, 1, 1000, 1000, 128, "bf16", True, (-1, -1), None, 215),
    ("group3_window_left", 1, 6, 2, 260, 260, 128, "bf16", True, (64, -1), None, 216),
    ("group6_d64_fp16", 1, 6, 1, 300, 333, 64, "fp16", False, (-1, -1), None, 217),
]


def run_case(case):
    name, B, Hq, Hkv, Sq, Sk, d, dt, causal, window, scale, seed = case
    q, k, v = synth.gen_padded(seed, B, Hq, Hkv, Sq, Sk, d, dt)
    go = synth.gen_grad(seed + 1000, q.shape, dt)
    qd, kd, vd, god = q.to(DEV), k.to(DEV), v.to(DEV), go.to(DEV)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, window=window, softmax_scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, god, lse, causal=causal, window=window,
                        softmax_scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, go), (dq, dk, dv)


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_matches_oracle(case):
    name = case[0]
    causal, window, scale = case[8], case[9], case[10]
    print(f"[case] bwd {case}", flush=True)
    (q, k, v, go), (dq, dk, dv) = run_case(case)
    rq, rk, rv = oracle.attention_bwd(q, k, v, go, causal=causal, window=window, scale=scale)
    bq, bk, bv = error_bounds(q, k, v, go, causal, window, scale)
    check(name + ".dq", dq, rq, bq)
    check(name + ".dk", dk, rk, bk)
    check(name + ".dv", dv, rv, bv)


def test_bwd_no_keys_gives_zero_dq():
    print("[case] bwd no keys", flush=True)
    q, k, v = synth.gen_padded(230, 1, 2, 2, 40, 0, 128, "bf16")
    go = synth.gen_grad(231, q.shape)
    qd = q.to(DEV)
    o, lse = fa.fwd(qd, k.to(DEV), v.to(DEV))
    dq, dk, dv = fa.bwd(qd, k.to(DEV), v.to(DEV), o, go.to(DEV), lse)
    torch.cuda.synchronize()
    assert dq.float().abs().max().item() == 0.0 and dk.numel() == 0 and dv.numel() == 0


def test_bwd_no_queries_gives_zero_dkdv():
    print("[case] bwd no queries", flush=True)
    q, k, v = synth.gen_padded(232, 1, 4, 2, 0, 100, 128, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qd)
    lse = torch.empty((1, 4, 0), dtype=torch.float32, device=DEV)
    dk = torch.full_like(kd, 7.0)
    dv = torch.full_like(vd, 7.0)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, torch.empty_like(qd), lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dk.float().abs().max().item() == 0.0 and dv.float().abs().max().item() == 0.0


def test_bwd_deterministic_bitwise():
    """No atomics: two calls on the same inputs give identical bits."""
    case = BWD_CASES[0]
    print(f"[case] bwd determinism {case[0]}", flush=True)
    _, g1 = run_case(case)
    _, g2 = run_case(case)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
