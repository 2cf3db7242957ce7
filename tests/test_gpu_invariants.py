"""GPU invariants that hold exactly for this path (bitwise) or within the
parity tolerance: run-to-run determinism, masked keys have no effect, GQA
equals MHA with repeated K/V heads, packed equals per-sequence, decode equals
the last row of a causal prefill, split size does not matter."""
import pytest
import torch

import oracle
from exact_attention_08_amd import fa, synth
from oracle.checks import compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_deterministic_bitwise():
    q, k, v = synth.gen_padded(501, 2, 8, 2, 700, 700, 128, "bf16")
    print("[case] determinism fwd", flush=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.fwd(qd, kd, vd, causal=True)
    o2, l2 = fa.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    q, kc, vc, sl = synth.gen_decode(502, 4, 8, 2, 128, 3000, 0, 0, "bf16",
                                     lengths=[3000, 17, 1024, 2049])
    print("[case] determinism decode", flush=True)
    args = (q.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV), 3000)
    a1 = fa.decode_kvcache(*args, split_size=256)
    a2 = fa.decode_kvcache(*args, split_size=256)
    torch.cuda.synchronize()
    assert torch.equal(a1[0], a2[0]) and torch.equal(a1[1], a2[1])


def test_masked_future_keys_have_no_effect():
    S, J0 = 600, 333
    q, k, v = synth.gen_padded(503, 1, 4, 2, S, S, 128, "bf16")
    k2, v2 = k.clone(), v.clone()
    k2[:, J0:] = 1e4
    v2[:, J0:] = -1e4
    print("[case] causal perturbation", flush=True)
    o1, l1 = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    o2, l2 = fa.fwd(q.to(DEV), k2.to(DEV), v2.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :J0], o2[:, :J0]) and torch.equal(l1[:, :, :J0], l2[:, :, :J0])


def test_keys_outside_window_have_no_effect():
    S, wl = 512, 64
    q, k, v = synth.gen_padded(504, 1, 2, 2, S, S, 128, "bf16")
    i0 = 400                         # rows >= i0 see keys >= i0 - wl only
    k2, v2 = k.clone(), v.clone()
    k2[:, :i0 - wl] = -1e4
    v2[:, :i0 - wl] = 1e4
    print("[case] window perturbation", flush=True)
    o1, l1 = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=(wl, 0))
    o2, l2 = fa.fwd(q.to(DEV), k2.to(DEV), v2.to(DEV), causal=True, window=(wl, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1[:, i0:], o2[:, i0:]) and torch.equal(l1[:, :, i0:], l2[:, :, i0:])


def test_other_sequences_have_no_effect():
    lens = [100, 300, 77]
    q, k, v, cu, _ = synth.gen_varlen(505, 3, 0, 0, 8, 2, 128, "bf16", lengths=lens)
    k2, v2 = k.clone(), v.clone()
    k2[100:400] = 1e4
    v2[100:400] = -1e4
    print("[case] varlen perturbation", flush=True)
    cud = cu.to(DEV)
    o1, l1 = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cud, cud, 300, 300, causal=True)
    o2, l2 = fa.fwd_varlen(q.to(DEV), k2.to(DEV), v2.to(DEV), cud, cud, 300, 300, causal=True)
    torch.cuda.synchronize()
    for a, b in ((0, 100), (400, 477)):
        assert torch.equal(o1[a:b], o2[a:b]) and torch.equal(l1[:, a:b], l2[:, a:b])


def test_cache_rows_past_length_have_no_effect():
    q, kc, vc, sl = synth.gen_decode(506, 2, 8, 2, 128, 2048, 0, 0, "bf16", lengths=[1000, 2048])
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[0, 1000:] = 1e4
    vc2[0, 1000:] = -1e4
    print("[case] decode perturbation", flush=True)
    a = fa.decode_kvcache(q.to(DEV), kc.to(DEV), vc.to(DEV), sl.to(DEV), 2048)
    b = fa.decode_kvcache(q.to(DEV), kc2.to(DEV), vc2.to(DEV), sl.to(DEV), 2048)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_gqa_equals_repeated_mha():
    q, k, v = synth.gen_padded(507, 2, 8, 2, 300, 300, 128, "bf16")
    print("[case] gqa vs mha", flush=True)
    o1, l1 = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    kr = k.repeat_interleave(4, dim=2).contiguous()
    vr = v.repeat_interleave(4, dim=2).contiguous()
    o2, l2 = fa.fwd(q.to(DEV), kr.to(DEV), vr.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_equals_per_sequence():
    lens = [129, 1, 300, 64]
    q, k, v, cu, _ = synth.gen_varlen(508, 4, 0, 0, 8, 2, 128, "bf16", lengths=lens)
    print("[case] varlen vs per-sequence", flush=True)
    cud = cu.to(DEV)
    o, l = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cud, cud, 300, 300, causal=True)
    torch.cuda.synchronize()
    for z in range(len(lens)):
        a, b = int(cu[z]), int(cu[z + 1])
        oz, lz = fa.fwd(q[None, a:b].contiguous().to(DEV), k[None, a:b].contiguous().to(DEV),
                        v[None, a:b].contiguous().to(DEV), causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], oz[0]) and torch.equal(l[:, a:b], lz[0])


def test_decode_equals_last_prefill_row_and_split_free():
    L, Hq, Hkv, d = 1500, 8, 2, 128
    q, k, v = synth.gen_padded(509, 1, Hq, Hkv, L, L, d, "bf16")
    kc = torch.zeros(1, 2048, Hkv, d, dtype=k.dtype)
    vc = torch.zeros(1, 2048, Hkv, d, dtype=k.dtype)
    kc[:, :L], vc[:, :L] = k, v
    sl = torch.tensor([L], dtype=torch.int32)
    print("[case] decode vs prefill", flush=True)
    o_pf, l_pf = fa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    qd = q[:, L - 1:L].contiguous().to(DEV)
    outs = [fa.decode_kvcache(qd, kc.to(DEV), vc.to(DEV), sl.to(DEV), L, split_size=s)
            for s in (64, 256, 1024, 2048)]
    torch.cuda.synchronize()
    ro, rl = oracle.attention_decode(q[:, L - 1:L], kc, vc, sl)
    for (o, lse) in outs:
        compare(o, lse, ro, rl, "bf16", "decode split")
        compare(o[:, 0], lse, o_pf[:, L - 1], l_pf[:, :, L - 1], "bf16", "decode vs prefill")
