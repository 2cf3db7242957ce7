"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and names workload shapes; it holds
none of the attention arithmetic, so both the GPU path and the fp64 oracle
can consume its outputs without sharing any of the method's code.

Recipe (the same everywhere):
  * a CPU ``torch.Generator`` seeded with the workload's seed;
  * draw order: sequence lengths (if any), then Q, then K, then V;
  * values are float32 N(0, sigma^2), then cast with round-to-nearest-even to
    the compute dtype (bf16 or fp16); the oracle reads the cast values;
  * KV-cache rows past a sequence's length are zero (never read).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """One named workload shape."""
    name: str
    kind: str                     # "fwd" | "varlen" | "decode"
    seed: int
    dtype: str = "bf16"
    B: int = 1
    Hq: int = 1
    Hkv: int = 1
    Sq: int = 0
    Sk: int = 0
    d: int = 128
    causal: bool = False
    window: tuple = (-1, -1)
    sigma: float = 1.0
    len_range: tuple = (0, 0)     # inclusive integer range for varlen / decode
    Sk_cap: int = 0               # decode cache capacity
    split: int = 1024             # decode split size
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.d ** -0.5


# The five workloads of the attention benchmark, sizes as stated there.
WORKLOADS = {
    "small_noncausal": Workload("small_noncausal", "fwd", seed=1, B=1, Hq=1, Hkv=1,
                                Sq=256, Sk=256, d=64),
    "causal_gqa_prefill": Workload("causal_gqa_prefill", "fwd", seed=2, B=4, Hq=32, Hkv=8,
                                   Sq=4096, Sk=4096, d=128, causal=True),
    "causal_window": Workload("causal_window", "fwd", seed=3, dtype="fp16", B=2, Hq=32,
                              Hkv=32, Sq=16384, Sk=16384, d=128, causal=True,
                              window=(256, 256), sigma=0.5),
    "varlen_causal": Workload("varlen_causal", "varlen", seed=4, B=64, Hq=32, Hkv=8,
                              d=128, causal=True, len_range=(32, 2048)),
    # keys per decode split: a sweep of 1024-3072 on this workload (the
    # split is the caller's choice) measured 2560 fastest, 1024 and 2048 2 %
    # slower (how evenly the splits' work-groups fill the GPU's last wave)
    "kvcache_decode": Workload("kvcache_decode", "decode", seed=5, B=64, Hq=32, Hkv=8,
                               d=128, len_range=(1024, 32768), Sk_cap=32768, split=2560),
    "long_causal_prefill": Workload("long_causal_prefill", "fwd", seed=50, B=1, Hq=32,
                                    Hkv=8, Sq=65536, Sk=65536, d=128, causal=True),
}


def _normal(gen: torch.Generator, shape, sigma: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def gen_padded(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int,
               dtype: str = "bf16", sigma: float = 1.0):
    """q: [B,Sq,Hq,d], k,v: [B,Sk,Hkv,d] on the CPU."""
    gen = torch.Generator().manual_seed(seed)
    t = DTYPES[dtype]
    q = _normal(gen, (B, Sq, Hq, d), sigma, t)
    k = _normal(gen, (B, Sk, Hkv, d), sigma, t)
    v = _normal(gen, (B, Sk, Hkv, d), sigma, t)
    return q, k, v


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor 8-bit e4m3 quantisation of a float tensor: descale =
    max|x| / 448 (the format's largest value), codes = RNE(x / descale) as
    torch's float8_e4m3fn cast, returned as uint8 with the fp32 descale."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = amax / 448.0 if amax > 0 else 1.0
    codes = (x.float() / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, float(torch.tensor(descale, dtype=torch.float32))


def gen_fp8(seed: int, B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, sigma: float = 1.0):
    """8-bit inputs: fp32 N(0, sigma^2) drawn as gen_padded draws them (Q, K,
    V in that order), each tensor quantised per tensor by quantize_e4m3.
    -> (q8, k8, v8) uint8 [B,S,H,d] and (descale_q, descale_k, descale_v)."""
    gen = torch.Generator().manual_seed(seed)
    xs = [_normal(gen, shape, sigma, torch.float32)
          for shape in ((B, Sq, Hq, d), (B, Sk, Hkv, d), (B, Sk, Hkv, d))]
    out = [quantize_e4m3(x) for x in xs]
    return tuple(c for c, _ in out), tuple(s for _, s in out)


def gen_grad(seed: int, shape, dtype: str = "bf16", sigma: float = 1.0) -> torch.Tensor:
    """A seeded incoming gradient (dL/dO) of the given shape, N(0, sigma^2)."""
    gen = torch.Generator().manual_seed(seed)
    return _normal(gen, tuple(shape), sigma, DTYPES[dtype])


def gen_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> torch.Tensor:
    """n integer lengths uniform in [lo, hi] (inclusive)."""
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)


def cumulative(lengths) -> torch.Tensor:
    """int32 cumulative lengths [0, l0, l0+l1, ...]."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu.to(torch.int32)


def gen_varlen(seed: int, nseq: int, lo: int, hi: int, Hq: int, Hkv: int, d: int,
               dtype: str = "bf16", sigma: float = 1.0, lengths=None):
    """Packed self-attention batch: q: [total,Hq,d], k,v: [total,Hkv,d],
    cu_seqlens int32 [nseq+1] (same for q and k), lengths int64 [nseq]."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = gen_lengths(gen, nseq, lo, hi)
    else:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
    total = int(lengths.sum())
    t = DTYPES[dtype]
    q = _normal(gen, (total, Hq, d), sigma, t)
    k = _normal(gen, (total, Hkv, d), sigma, t)
    v = _normal(gen, (total, Hkv, d), sigma, t)
    return q, k, v, cumulative(lengths), lengths


def gen_decode(seed: int, B: int, Hq: int, Hkv: int, d: int, Sk_cap: int, lo: int, hi: int,
               dtype: str = "bf16", sigma: float = 1.0, lengths=None):
    """q: [B,1,Hq,d]; k_cache, v_cache: [B,Sk_cap,Hkv,d] (rows past each
    length are zero); cache_seqlens int32 [B].  Cache rows are drawn one
    sequence at a time (K for all sequences, then V) to bound host memory."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = gen_lengths(gen, B, lo, hi)
    else:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
    t = DTYPES[dtype]
    q = _normal(gen, (B, 1, Hq, d), sigma, t)
    kc = torch.zeros((B, Sk_cap, Hkv, d), dtype=t)
    vc = torch.zeros((B, Sk_cap, Hkv, d), dtype=t)
    for cache in (kc, vc):
        for b in range(B):
            L = int(lengths[b])
            cache[b, :L] = _normal(gen, (L, Hkv, d), sigma, t)
    return q, kc, vc, lengths.to(torch.int32)


def gen_paged(seed: int, B: int, Hq: int, Hkv: int, d: int, page_size: int, lo: int, hi: int,
              dtype: str = "bf16", sigma: float = 1.0, lengths=None, append: bool = True,
              spare_pages: int = 0):
    """Paged-cache decode inputs.  Sequence b has lengths[b] keys in all; with
    ``append`` the cache holds the first lengths[b] - 1 and the last one is
    the new token (k_new, v_new), otherwise the cache holds all of them.
    Lengths, Q, K and V are drawn exactly as gen_decode draws them (same
    seed, same values).  The pool has sum(ceil(len / page_size)) +
    spare_pages pages; their order is a random permutation from a second
    generator seeded with seed + 7919, each sequence taking the next
    ceil(len / page_size) of it.  Rows of a page past a sequence's cached
    rows, and spare pages, are zero.
    -> q [B,1,Hq,d], k_pages, v_pages [num_pages,page_size,Hkv,d],
       block_table int32 [B,max_pages], cache_seqlens int32 [B],
       k_new, v_new [B,1,Hkv,d] (None without append), lengths int64 [B]."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = gen_lengths(gen, B, lo, hi)
    else:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
    t = DTYPES[dtype]
    need = [-(-int(n) // page_size) for n in lengths]
    max_pages = max(max(need), 1)
    num_pages = sum(need) + spare_pages
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed + 7919))
    table = torch.zeros((B, max_pages), dtype=torch.int32)
    nxt = 0
    for b in range(B):
        table[b, :need[b]] = perm[nxt:nxt + need[b]].to(torch.int32)
        nxt += need[b]
    cached = lengths - 1 if append else lengths
    q = _normal(gen, (B, 1, Hq, d), sigma, t)
    pools, new = {}, {}
    for w in ("k", "v"):
        pool = torch.zeros((num_pages, page_size, Hkv, d), dtype=t)
        last = torch.zeros((B, 1, Hkv, d), dtype=t)
        for b in range(B):
            L, n_cached = int(lengths[b]), int(cached[b])
            rows = _normal(gen, (L, Hkv, d), sigma, t)
            if L > 0:
                last[b, 0] = rows[L - 1]
            for pg in range(need[b]):
                a, e = pg * page_size, min((pg + 1) * page_size, n_cached)
                if e > a:
                    pool[int(table[b, pg]), :e - a] = rows[a:e]
        pools[w], new[w] = pool, last
    k_new, v_new = (new["k"], new["v"]) if append else (None, None)
    return (q, pools["k"], pools["v"], table, cached.to(torch.int32), k_new, v_new, lengths)


def generate(w: Workload):
    """Inputs of a named workload (CPU tensors)."""
    if w.kind == "fwd":
        return gen_padded(w.seed, w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.dtype, w.sigma)
    if w.kind == "varlen":
        return gen_varlen(w.seed, w.B, w.len_range[0], w.len_range[1], w.Hq, w.Hkv, w.d,
                          w.dtype, w.sigma)
    if w.kind == "decode":
        return gen_decode(w.seed, w.B, w.Hq, w.Hkv, w.d, w.Sk_cap, w.len_range[0],
                          w.len_range[1], w.dtype, w.sigma)
    raise ValueError(w.kind)
