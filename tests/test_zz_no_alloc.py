"""The allocation-free decode entry point (fa_decode_kvcache_noalloc): the
same results as fa_decode_kvcache with a caller workspace, on two calls in a
row (the second smaller, so stale partials of the first would show), and
sizes beyond its scratch array rejected on the host."""
import pytest
import torch

from exact_attention_08_amd import fa, synth

pytestmark = pytest.mark.gpu


def _run_both(seed, B, Hq, Hkv, d, cap, lengths, split, dtype, stream=None):
    q, kc, vc, sl = synth.gen_decode(seed, B, Hq, Hkv, d, cap, 0, 0, dtype, lengths=lengths)
    dev = "cuda:0"
    q, kc, vc, sl = q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev)
    L = max(lengths)
    ref_o, ref_l = fa.decode_kvcache(q, kc, vc, sl, L, split_size=split)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if stream is None:
        fa.decode_kvcache_noalloc(q, kc, vc, sl, L, out=out, lse=lse, split_size=split)
    else:
        with torch.cuda.stream(stream):
            fa.decode_kvcache_noalloc(q, kc, vc, sl, L, out=out, lse=lse, split_size=split)
        stream.synchronize()
    torch.cuda.synchronize()
    print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} d={d} split={split} max_len={L}", flush=True)
    return out, lse, ref_o, ref_l


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: 8 sequences, up to 9000 keys, 1024-key splits (9 per row)
    lens1 = [9000, 1, 4097, 2048, 777, 8191, 3000, 64]
    o1, l1, r1, rl1 = _run_both(301, 8, 32, 8, 128, 9000, lens1, 1024, "bf16")
    assert torch.equal(o1, r1) and torch.equal(l1, rl1)
    # second call, smaller: fewer sequences, other head shape and split size
    lens2 = [700, 1500, 129]
    o2, l2, r2, rl2 = _run_both(302, 3, 8, 2, 64, 1500, lens2, 512, "fp16")
    assert torch.equal(o2, r2) and torch.equal(l2, rl2)


def test_noalloc_on_a_side_stream():
    s = torch.cuda.Stream()
    o, l, r, rl = _run_both(303, 4, 16, 4, 128, 5000, [5000, 2500, 33, 4096], 1024, "bf16",
                            stream=s)
    assert torch.equal(o, r) and torch.equal(l, rl)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # 64 sequences x 32 heads x 64 splits x 129 fp32 > 64 MiB: rejected on the host
    B, Hq, Hkv, d = 64, 32, 8, 128
    need = fa.decode_workspace_bytes(B, Hq, 65536, d, 1024)
    assert need > fa.DECODE_NOALLOC_MAX_BYTES
    lib = fa.load()
    st = lib.fa_decode_kvcache_noalloc(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None,
                                       B, Hq, Hkv, 65536, 65536, d, 1, -1, -1, 0.088, 1024, 0, None)
    assert st == 3
    assert "scratch" in lib.fa_last_error().decode()
