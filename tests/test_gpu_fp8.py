"""GPU parity of the 8-bit forward (fa_fwd_fp8 through the C ABI) against
the fp64 oracle on the exact values the 8-bit codes stand for.

Tolerance, derived from the arithmetic: the scores and every sum are fp32
(LSE within 1e-3, as for the 16-bit forward), but the weights enter P.V
rounded to e4m3.  Under the lazy max each weight is w = 2^(u - m) with the
running max m at most the row's true max, so w is at least p * L0 with
L0 = sum_j exp(s_j - max s) >= 1 (p the exact probabilities).  RNE to e4m3
moves a weight by at most 2^-4 w (normal range) or 2^-10 (the subnormal
spacing is 2^-9), and never by more than w itself when it rounds to zero.
O divides by the fp32 sum of the unrounded weights, so per element
    |dO_ic| <= sum_j max(2^-4 p_ij, min(p_ij, 2^-10 / L0_i)) |v_jc|
plus 2^-8 |O_ic| for the bf16 output and 1e-5 for fp32 rounding."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, B, Hq, Hkv, Sq, Sk, d, causal, window, scale, sigma, seed
FP8_CASES = [
    ("causal_gqa_ragged", 2, 8, 2, 300, 300, 128, True, (-1, -1), None, 1.0, 701),
    ("noncausal_d64_ragged", 2, 4, 1, 130, 257, 64, False, (-1, -1), None, 1.0, 702),
    ("window_causal", 1, 4, 4, 400, 400, 128, True, (100, 100), None, 1.0, 703),
    ("causal_sq_lt_sk", 1, 4, 2, 77, 300, 128, True, (-1, -1), None, 1.0, 704),
    ("causal_sq_gt_sk", 1, 4, 2, 300, 77, 128, True, (-1, -1), None, 1.0, 705),
    ("negative_scale", 1, 2, 2, 150, 150, 128, True, (-1, -1), -0.09, 1.0, 706),
    ("large_scores", 1, 4, 2, 256, 256, 128, True, (-1, -1), 0.5, 1.0, 707),
    ("long_causal", 1, 4, 1, 1000, 1000, 128, True, (-1, -1), None, 1.0, 708),
    ("window_two_sided_d64", 1, 2, 1, 300, 300, 64, False, (50, 30), None, 1.0, 709),
    ("single_key", 1, 2, 2, 50, 1, 128, False, (-1, -1), None, 1.0, 710),
    ("group3", 1, 6, 2, 200, 200, 128, True, (-1, -1), None, 1.0, 712),
    ("group16", 1, 16, 1, 130, 130, 128, True, (-1, -1), None, 1.0, 713),
    ("d64_causal_gqa", 2, 8, 2, 300, 300, 64, True, (-1, -1), None, 1.0, 714),
    ("window_left_long", 1, 4, 4, 700, 700, 128, True, (200, -1), None, 0.5, 715),
    # rows that see more than 2560 keys on average: the wide (64-row) form;
    # the cases above run on the paired (32-row) form
    ("wide_causal", 1, 4, 1, 5300, 5300, 128, True, (-1, -1), None, 1.0, 716),
    ("wide_noncausal_d64", 1, 2, 1, 100, 2700, 64, False, (-1, -1), None, 1.0, 717),
    ("wide_window_two_sided", 1, 2, 2, 200, 3000, 128, False, (1500, 1100), None, 1.0, 718),
]


def fp8_bounds(q, k, v, causal, window, scale):
    """Per-element bound of |O_gpu - O_ref| (see the module docstring) from
    the exact (decoded, descaled) fp64 inputs; tolerances only."""
    from oracle_pins import _visible_band
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    vis = _visible_band(Sq, Sk, causal, window[0], window[1]).numpy()
    bound = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            s = np.where(vis, scale * q[b, :, h] @ k[b, :, h // G].T, -np.inf)
            m = s.max(1, keepdims=True)
            m[~np.isfinite(m)] = 0.0
            e = np.where(vis, np.exp(s - m), 0.0)
            L0 = e.sum(1, keepdims=True)
            p = e / np.where(L0 > 0, L0, 1.0)
            wabs = np.maximum(2.0 ** -4 * p, np.minimum(p, 2.0 ** -10 / np.where(L0 > 0, L0, 1.0)))
            bound[b, :, h] = wabs @ np.abs(v[b, :, h // G])
    return bound


def run(case):
    name, B, Hq, Hkv, Sq, Sk, d, causal, window, scale, sigma, seed = case
    (q8, k8, v8), (dq, dk, dv) = synth.gen_fp8(seed, B, Hq, Hkv, Sq, Sk, d, sigma)
    o, lse = fa.fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), dq, dk, dv, causal=causal, window=window,
                        softmax_scale=scale)
    torch.cuda.synchronize()
    return (q8, k8, v8, dq, dk, dv), o, lse


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_matches_oracle(case):
    name, B, Hq, Hkv, Sq, Sk, d, causal, window, scale, sigma, seed = case
    print(f"[case] fp8 {case}", flush=True)
    (q8, k8, v8, dq, dk, dv), o, lse = run(case)
    sc = scale if scale is not None else d ** -0.5
    ro, rl = oracle.attention_fp8(q8, k8, v8, dq, dk, dv, causal=causal, window=window, scale=sc)
    og = o.to("cpu", torch.float64).numpy()
    lg = lse.cpu().double().numpy()
    assert np.isfinite(og).all()
    qf = oracle.decode_e4m3(q8) * dq
    kf = oracle.decode_e4m3(k8) * dk
    vf = oracle.decode_e4m3(v8) * dv
    tol = fp8_bounds(qf, kf, vf, causal, window, sc) + 2.0 ** -8 * np.abs(ro) + 1e-5
    err = np.abs(og - ro)
    worst = float((err / tol).max()) if err.size else 0.0
    ninf = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lg), ninf), f"{name}: -inf LSE pattern differs"
    dl = float(np.abs(lg[~ninf] - rl[~ninf]).max()) if (~ninf).any() else 0.0
    print(f"[parity] fp8 {name}: max|dO| {err.max():.4g} (worst err/bound {worst:.3f}, "
          f"rms err {np.sqrt((err ** 2).mean()):.3g}), max|dLSE| {dl:.3g}", flush=True)
    assert (err <= tol).all(), f"{name}: {int((err > tol).sum())} outputs exceed the bound"
    assert dl <= 1e-3, f"{name}: max |dLSE| {dl:.3g} > 1e-3"


def test_fp8_no_keys():
    print("[case] fp8 no keys", flush=True)
    case = ("no_keys", 1, 2, 2, 40, 0, 128, True, (-1, -1), None, 1.0, 711)
    _, o, lse = run(case)
    assert o.float().abs().max().item() == 0.0 and torch.isneginf(lse).all()
