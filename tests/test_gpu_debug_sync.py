"""The checking build of the library (libfa355_debug.so: every copy-pipeline
wait drains all outstanding copies, the forward and backward kernels fill
their LDS rings with NaN before the first copy) against the pipelined build,
bit for bit, on every entry point.  A tile read before its copy had landed,
or LDS bytes read that no copy writes, would make the two differ (NaN in the
checking build, or other values): this checks the hand-counted copy waits of
the pipelines independently of the oracle."""
import pytest
import torch

from exact_attention_08_amd import fa, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(fn):
    """fn() on the pipelined library, then on the checking library."""
    a = fn()
    torch.cuda.synchronize()
    with fa.using(fa.DEBUG_LIB_PATH):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def _equal(a, b, name):
    for x, y in zip(a, b):
        assert not torch.isnan(y.float()).any(), f"{name}: NaN in the checking build"
        assert torch.equal(x, y), f"{name}: results differ from the checking build"


# B, Hq, Hkv, Sq, Sk, d, dtype, causal, window: both forward kernels (rows that
# see up to 2,560 keys on average / more), ragged tails, windows, d = 64
FWD = [
    (2, 8, 2, 300, 300, 128, "bf16", True, (-1, -1)),
    (1, 4, 4, 700, 700, 128, "fp16", True, (100, 100)),
    (2, 4, 1, 130, 257, 64, "bf16", False, (-1, -1)),
    (1, 8, 2, 2200, 2200, 128, "bf16", True, (-1, -1)),
    (1, 8, 2, 5300, 5300, 128, "bf16", True, (-1, -1)),
    (1, 4, 2, 300, 2900, 64, "fp16", True, (-1, -1)),
]


@pytest.mark.parametrize("case", FWD, ids=[f"fwd{i}" for i in range(len(FWD))])
def test_forward_checking_build(case):
    B, Hq, Hkv, Sq, Sk, d, dt, causal, window = case
    print(f"[case] checking build fwd {case}", flush=True)
    q, k, v = (x.to(DEV) for x in synth.gen_padded(701, B, Hq, Hkv, Sq, Sk, d, dt))
    a, b = _both(lambda: fa.fwd(q, k, v, causal=causal, window=window))
    _equal(a, b, f"fwd {case}")


def test_varlen_checking_build():
    print("[case] checking build varlen", flush=True)
    lens = [1, 127, 300, 0, 5400, 64]
    q, k, v, cu, _ = synth.gen_varlen(702, len(lens), 0, 0, 8, 2, 128, "bf16", lengths=lens)
    q, k, v, cu = q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV)
    for mx in (300, max(lens)):           # the paired kernel, then the wide one
        sub = [min(x, mx) for x in lens]
        cs = synth.cumulative(sub).to(DEV)
        n = int(sum(sub))
        a, b = _both(lambda: fa.fwd_varlen(q[:n], k[:n], v[:n], cs, cs, mx, mx, causal=True))
        _equal(a, b, f"varlen max {mx}")
    del cu


def test_modifiers_checking_build():
    print("[case] checking build fwd_mod", flush=True)
    q, k, v = (x.to(DEV) for x in synth.gen_padded(703, 1, 8, 2, 400, 400, 128, "bf16"))
    slopes = torch.tensor([2.0 ** (-(h + 1)) for h in range(8)], device=DEV)
    a, b = _both(lambda: fa.fwd_mod(q, k, v, causal=True, alibi_slopes=slopes, softcap=30.0))
    _equal(a, b, "fwd_mod")


def test_fp8_checking_build():
    print("[case] checking build fwd_fp8", flush=True)
    (q8, k8, v8), (dq, dk, dv) = synth.gen_fp8(704, 1, 8, 2, 300, 300, 128)
    q8, k8, v8 = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    a, b = _both(lambda: fa.fwd_fp8(q8, k8, v8, dq, dk, dv, causal=True))
    _equal(a, b, "fwd_fp8")


def test_decode_checking_build():
    print("[case] checking build decode", flush=True)
    q, kc, vc, sl = synth.gen_decode(705, 4, 8, 2, 128, 2600, 0, 0, "bf16",
                                     lengths=[1, 700, 2600, 1025])
    q, kc, vc, sl = q.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV)
    a, b = _both(lambda: fa.decode_kvcache(q, kc, vc, sl, 2600, split_size=512))
    _equal(a, b, "decode")


def test_paged_checking_build():
    print("[case] checking build paged decode", flush=True)
    q, kp, vp, bt, sl, kn, vn, lens = synth.gen_paged(706, 3, 8, 2, 128, 64, 0, 0, "bf16",
                                                      lengths=[100, 1000, 65], append=True)
    q, bt, sl, kn, vn = q.to(DEV), bt.to(DEV), sl.to(DEV), kn.to(DEV), vn.to(DEV)
    kp1, vp1, kp2, vp2 = kp.to(DEV), vp.to(DEV), kp.to(DEV), vp.to(DEV)
    o1, l1 = fa.decode_paged(q, kp1, vp1, bt, sl, int(max(lens)), k_new=kn, v_new=vn,
                             split_size=256)
    torch.cuda.synchronize()
    with fa.using(fa.DEBUG_LIB_PATH):
        o2, l2 = fa.decode_paged(q, kp2, vp2, bt, sl, int(max(lens)), k_new=kn, v_new=vn,
                                 split_size=256)
        torch.cuda.synchronize()
    _equal((o1, l1, kp1, vp1), (o2, l2, kp2, vp2), "paged decode")


def test_backward_checking_build():
    print("[case] checking build bwd", flush=True)
    q, k, v = (x.to(DEV) for x in synth.gen_padded(707, 2, 8, 2, 300, 333, 128, "bf16"))
    go = synth.gen_grad(708, q.shape).to(DEV)
    o, lse = fa.fwd(q, k, v, causal=True)
    a, b = _both(lambda: fa.bwd(q, k, v, o, go, lse, causal=True))
    _equal(a, b, "bwd")
