"""The comparison helpers of oracle/checks.py on hand-made values (CPU only):
the one-ulp rule of compare()."""
import numpy as np
import torch

from oracle.checks import compare, ulp


def test_ulp_of_bf16_and_fp16():
    assert ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert ulp(np.array([3.0]), "bf16")[0] == 2.0 ** -6
    assert ulp(np.array([1.0]), "fp16")[0] == 2.0 ** -10


def test_compare_accepts_one_ulp_above_tolerance_only_for_large_values():
    ref_o = np.array([[3.0 + 2 ** -7]])           # exact value between two bf16 numbers
    ref_l = np.array([0.0])
    o_ok = torch.tensor([[3.0 + 2 ** -6]], dtype=torch.bfloat16)    # err 2^-7 < 1e-2
    st = compare(o_ok, torch.tensor([0.0]), ref_o, ref_l, "bf16", "ok")
    assert st["n_over_1e-2"] == 0
    o_far = torch.tensor([[3.0 + 2 ** -5]], dtype=torch.bfloat16)   # err 0.0234, > one ulp
    try:
        compare(o_far, torch.tensor([0.0]), ref_o, ref_l, "bf16", "far")
    except AssertionError:
        pass
    else:
        raise AssertionError("an error beyond one ulp and 1e-2 must fail")
