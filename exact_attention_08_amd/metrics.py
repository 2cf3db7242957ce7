"""Algorithmic work of an attention call, for throughput accounting.

FLOP = 4*d per visible (query, key) pair per query head (2*d for the score
dot product, 2*d for the weighted sum of values): the work the method itself
must do, excluding softmax arithmetic, masked lanes inside boundary tiles and
padding.  Bytes = Q, K, V read once and O, LSE written once; for decode only
the cache rows that are visible.  MI355X peaks are the published figures.
"""
from __future__ import annotations

import numpy as np

PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA, 256 CU x 2.4 GHz x 8192 FLOP/clk
PEAK_BF16_TFLOPS = 2516.6      # dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0          # HBM3E


def visible_pairs(Sq: int, Sk: int, causal: bool, window=(-1, -1)) -> int:
    """Number of visible (i, j) pairs of one (sequence, head), bottom-right
    aligned, inclusive window bounds (-1 = unbounded)."""
    if Sq <= 0 or Sk <= 0:
        return 0
    i = np.arange(Sq, dtype=np.int64)
    pos = i + (Sk - Sq)
    hi = np.full(Sq, Sk - 1, dtype=np.int64)
    lo = np.zeros(Sq, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, pos)
    if window[1] >= 0:
        hi = np.minimum(hi, pos + window[1])
    if window[0] >= 0:
        lo = np.maximum(lo, pos - window[0])
    return int(np.maximum(hi - lo + 1, 0).sum())


def fwd_work(B, Hq, Hkv, Sq, Sk, d, causal, window=(-1, -1), elem_bytes=2):
    pairs = B * Hq * visible_pairs(Sq, Sk, causal, window)
    flop = 4 * d * pairs
    byts = elem_bytes * d * (2 * B * Sq * Hq + 2 * B * Sk * Hkv) + 4 * B * Hq * Sq
    return {"pairs": pairs, "flop": flop, "bytes": byts}


def bwd_work(B, Hq, Hkv, Sq, Sk, d, causal, window=(-1, -1), elem_bytes=2):
    """Gradients: five products of 2*d FLOP per visible (query, key) pair per
    query head (S = Q K^T recomputed, dP = dO V^T, dV += P^T dO,
    dK += dS^T Q, dQ += dS K), i.e. 2.5x the forward; bytes = Q, K, V, O, dO
    and LSE read once and dQ, dK, dV written once."""
    pairs = visible_pairs(Sq, Sk, causal, window)
    flop = 10 * d * pairs * B * Hq
    byts = (4 * B * Sq * Hq * d + 4 * B * Sk * Hkv * d) * elem_bytes + B * Hq * Sq * 4
    return {"flop": flop, "bytes": byts, "pairs": pairs * B * Hq}


def varlen_work(lengths_q, lengths_k, Hq, Hkv, d, causal, window=(-1, -1), elem_bytes=2):
    pairs = sum(Hq * visible_pairs(int(a), int(b), causal, window)
                for a, b in zip(lengths_q, lengths_k))
    tq, tk = int(np.sum(lengths_q)), int(np.sum(lengths_k))
    flop = 4 * d * pairs
    byts = elem_bytes * d * (2 * tq * Hq + 2 * tk * Hkv) + 4 * Hq * tq
    return {"pairs": pairs, "flop": flop, "bytes": byts}


def decode_work(lengths, Hq, Hkv, d, window=(-1, -1), elem_bytes=2):
    lens = np.asarray(lengths, dtype=np.int64)
    if window[0] >= 0:
        vis = np.minimum(lens, window[0] + 1)
    else:
        vis = lens
    B = lens.size
    pairs = int(vis.sum()) * Hq
    flop = 4 * d * pairs
    byts = elem_bytes * d * (2 * int(vis.sum()) * Hkv + 2 * B * Hq) + 4 * B * Hq
    return {"pairs": pairs, "flop": flop, "bytes": byts}
