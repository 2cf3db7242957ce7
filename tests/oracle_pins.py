"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself.

Each pin is a function ``pin_x(orc)`` taking an ``oracle.Oracle`` and raising
AssertionError when the oracle disagrees with

  * the numbers the FlashAttention explainer page prints for its worked
    online-softmax example (golden fixture);
  * closed forms (zero queries give uniform weights, so LSE = ln(#visible)
    and O = mean of the visible value rows; constant V; one visible key);
  * a library routine (torch's float64 CPU scaled_dot_product_attention and
    logsumexp, with masks built independently from torch.tril/triu bands);
  * invariants of the definition (masked keys have no effect, key
    permutation, GQA equals MHA with repeated K/V heads, packed equals
    per-sequence, decode equals the last prefill row, key translation,
    split-and-combine by LSE);
  * a 30-digit mpmath brute force on tiny inputs;
  * for the gradients: central finite differences through the forward
    oracle, torch float64 autograd of an explicit masked softmax, and exact
    identities (row weights sum to one, key-translation invariance).

The functions are shared by ``test_oracle_pins.py`` (the real oracle) and
``test_oracle_mutations.py`` (deliberately broken copies of the oracle, each
of which must fail at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _visible_band(Sq, Sk, causal, wl, wr):
    """Boolean [Sq,Sk] visibility built from torch band helpers (independent
    of the oracle's predicate): query i sits at key position i + Sk - Sq."""
    delta = Sk - Sq
    m = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        m &= torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=delta)
    if wr >= 0:
        m &= torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=delta + wr)
    if wl >= 0:
        m &= torch.ones(Sq, Sk, dtype=torch.bool).triu(diagonal=delta - wl)
    return m


def _sdpa_reference(q, k, v, causal, wl, wr, scale):
    """torch float64 SDPA with an explicit mask; q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d]."""
    q = torch.from_numpy(q).permute(0, 2, 1, 3)
    k = torch.from_numpy(k).permute(0, 2, 1, 3)
    v = torch.from_numpy(v).permute(0, 2, 1, 3)
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    mask = _visible_band(q.shape[2], k.shape[2], causal, wl, wr)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                           scale=scale)
    s = (q @ k.transpose(-1, -2)) * scale
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


# ---------------------------------------------------------------------------
def pin_worked_example(orc):
    """Worked example of the explainer page: scores (1,3,2,5) split [1,3]|[2,5]."""
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    s = np.array(g["scores"])
    half = 0.5 * 10 ** -g["printed_decimals"]
    n = len(s)
    # q = e0, k_j = s_j e0, scale 1 -> scores s; V = identity so O row = P row.
    d = 4
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, d)); k[0, :, 0, 0] = s
    v = np.eye(n, d).reshape(1, n, 1, d)
    out, lse = orc.attention(q, k, v, scale=1.0)
    lse = lse[0, 0, 0]
    mx = g["direct"]["max"]
    assert abs(math.exp(lse - mx) - g["direct"]["sum"]) <= half
    # blocked sum: two rounded addends on the page
    assert abs(math.exp(lse - mx) - g["blocked_final_sum"]) <= 2 * half + 1e-12
    p = out[0, 0, 0, :n]
    assert abs(p.sum() - 1.0) < 1e-14
    for pj, ej in zip(p, g["direct"]["exps"]):
        assert abs(pj * math.exp(lse - mx) - ej) <= half
    # the two blocks on their own
    lses = []
    for (a, b), blk in zip(g["blocks"], (g["block1"], g["block2"])):
        _, l_b = orc.attention(q, k[:, a:b], v[:, a:b], scale=1.0)
        l_b = l_b[0, 0, 0]
        assert abs(math.exp(l_b - blk["max"]) - blk["sum"]) <= half
        lses.append(l_b)
    # rescaling of block one's sum to block two's max
    assert abs(math.exp(g["block1"]["max"] - g["block2"]["max"])
               - g["block2"]["old_sum_rescale"]) <= half
    assert abs(math.exp(lses[0] - g["block2"]["max"]) - g["block2"]["old_sum_rescaled"]) <= half
    # combining the block LSEs gives the full LSE
    M = max(lses)
    comb = M + math.log(sum(math.exp(x - M) for x in lses))
    assert abs(comb - lse) < 1e-12


def pin_torch_sdpa(orc):
    """Agreement with torch float64 SDPA + logsumexp for every mask mode."""
    rng = _rng(11)
    cases = [  # B, Hq, Hkv, Sq, Sk, d, causal, wl, wr, scale
        (2, 4, 2, 13, 13, 8, False, -1, -1, 0.37),
        (2, 4, 2, 13, 13, 8, True, -1, -1, 0.37),
        (1, 6, 3, 5, 13, 8, True, -1, -1, 0.5),
        (1, 2, 1, 11, 11, 5, False, 3, 2, 0.8),
        (1, 2, 2, 11, 11, 5, True, 3, 0, 0.8),
        (1, 3, 1, 7, 12, 4, False, 2, 4, 1.1),
        (1, 4, 4, 9, 9, 6, True, 4, 7, -0.3),
    ]
    for (B, Hq, Hkv, Sq, Sk, d, causal, wl, wr, scale) in cases:
        q = _rand(rng, B, Sq, Hq, d)
        k = _rand(rng, B, Sk, Hkv, d)
        v = _rand(rng, B, Sk, Hkv, d)
        out, lse = orc.attention(q, k, v, causal=causal, window=(wl, wr), scale=scale)
        ro, rl = _sdpa_reference(q, k, v, causal, wl, wr, scale)
        assert np.abs(out - ro).max() < 1e-12, (B, Hq, Hkv, Sq, Sk, causal, wl, wr)
        assert np.abs(lse - rl).max() < 1e-12, (B, Hq, Hkv, Sq, Sk, causal, wl, wr)


def _interval(i, Sq, Sk, causal, wl, wr):
    """Closed form of the visible key interval [lo, hi] of query row i."""
    pos = i + Sk - Sq
    lo, hi = 0, Sk - 1
    if causal:
        hi = min(hi, pos)
    if wr >= 0:
        hi = min(hi, pos + wr)
    if wl >= 0:
        lo = max(lo, pos - wl)
    return lo, hi


def pin_zero_query_closed_form(orc):
    """Q = 0: every visible key gets equal weight, so LSE = ln(#visible) and
    O = mean of the visible value rows."""
    rng = _rng(12)
    cases = [  # Sq, Sk, causal, wl, wr
        (10, 10, False, -1, -1), (10, 10, True, -1, -1), (6, 10, True, -1, -1),
        (12, 12, True, 3, 0), (12, 12, True, 3, 3), (12, 12, False, 2, 3),
        (7, 12, False, 0, 2), (12, 12, True, 0, 0), (9, 9, False, 4, 0),
    ]
    for (Sq, Sk, causal, wl, wr) in cases:
        d = 3
        q = np.zeros((1, Sq, 1, d))
        k = _rand(rng, 1, Sk, 1, d)
        v = _rand(rng, 1, Sk, 1, d)
        out, lse = orc.attention(q, k, v, causal=causal, window=(wl, wr), scale=0.9)
        for i in range(Sq):
            lo, hi = _interval(i, Sq, Sk, causal, wl, wr)
            cnt = hi - lo + 1
            assert cnt >= 1
            assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-13, (Sq, Sk, causal, wl, wr, i)
            assert np.abs(out[0, i, 0] - v[0, lo:hi + 1, 0].mean(0)).max() < 1e-13


def pin_varlen_zero_query(orc):
    """Packed sequences with Q = 0: LSE of local row i is ln(i+1) (causal),
    so no row may see another sequence's keys."""
    rng = _rng(13)
    lens = [3, 1, 6, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, d = int(cu[-1]), 4
    q = np.zeros((T, 2, d))
    k = _rand(rng, T, 1, d)
    v = _rand(rng, T, 1, d)
    out, lse = orc.attention_varlen(q, k, v, cu, cu, causal=True, scale=1.0)
    for z, L in enumerate(lens):
        for i in range(L):
            t = cu[z] + i
            for h in range(2):
                assert abs(lse[h, t] - math.log(i + 1)) < 1e-13
                assert np.abs(out[t, h] - v[cu[z]:t + 1, 0].mean(0)).max() < 1e-13


def pin_decode_zero_query(orc):
    """Decode with Q = 0: LSE = ln(cache length), O = mean of the cached V rows."""
    rng = _rng(14)
    B, cap, d = 3, 9, 4
    lens = np.array([9, 1, 5], dtype=np.int32)
    q = np.zeros((B, 1, 4, d))
    kc = _rand(rng, B, cap, 2, d)
    vc = _rand(rng, B, cap, 2, d)
    out, lse = orc.attention_decode(q, kc, vc, lens, causal=True)
    for b in range(B):
        for h in range(4):
            assert abs(lse[b, h] - math.log(lens[b])) < 1e-13
            assert np.abs(out[b, 0, h] - vc[b, :lens[b], h // 2].mean(0)).max() < 1e-13


def pin_constant_v(orc):
    """v_j = u for all j gives O = u for every row and mask mode."""
    rng = _rng(15)
    u = _rand(rng, 5)
    for (causal, wl, wr) in [(False, -1, -1), (True, -1, -1), (True, 2, 0), (False, 1, 3)]:
        q = _rand(rng, 2, 8, 2, 5)
        k = _rand(rng, 2, 8, 1, 5)
        v = np.broadcast_to(u, (2, 8, 1, 5)).copy()
        out, _ = orc.attention(q, k, v, causal=causal, window=(wl, wr), scale=0.7)
        assert np.abs(out - u).max() < 1e-14


def pin_single_visible_key(orc):
    """Causal with window (0,0): each row sees only its own key, so O_i = v_i
    and LSE_i = scale * q_i . k_i; causal row 0 also sees only key 0."""
    rng = _rng(16)
    q = _rand(rng, 1, 7, 2, 6)
    k = _rand(rng, 1, 7, 2, 6)
    v = _rand(rng, 1, 7, 2, 6)
    out, lse = orc.attention(q, k, v, causal=True, window=(0, 0), scale=0.6)
    assert np.array_equal(out, v)
    s = 0.6 * np.einsum("bshd,bshd->bhs", q, k)
    assert np.abs(lse - s).max() < 1e-14
    out2, lse2 = orc.attention(q, k, v, causal=True, scale=0.6)
    assert np.array_equal(out2[:, 0], v[:, 0])
    assert np.abs(lse2[:, :, 0] - s[:, :, 0]).max() < 1e-14


def pin_one_hot_values(orc):
    """v_j = e_j (Sk <= d): the output row is the probability row; it sums to 1
    and equals scipy's softmax of the scaled scores."""
    from scipy.special import softmax
    rng = _rng(17)
    Sk, d = 6, 8
    q = _rand(rng, 1, 5, 1, d)
    k = _rand(rng, 1, Sk, 1, d)
    v = np.eye(Sk, d).reshape(1, Sk, 1, d)
    out, _ = orc.attention(q, k, v, scale=0.45)
    p = softmax(0.45 * (q[0, :, 0] @ k[0, :, 0].T), axis=-1)
    assert np.abs(out[0, :, 0, :Sk] - p).max() < 1e-14
    assert np.abs(out[0, :, 0].sum(-1) - 1.0).max() < 1e-14
    assert np.all(out[0, :, 0, Sk:] == 0)


def pin_masked_keys_no_effect(orc):
    """Keys a row cannot see (future, outside the window, other sequences,
    past the cache length) may hold anything finite: the row is unchanged."""
    rng = _rng(18)
    Sq = Sk = 10
    q = _rand(rng, 1, Sq, 2, 4)
    k = _rand(rng, 1, Sk, 1, 4)
    v = _rand(rng, 1, Sk, 1, 4)
    for (causal, wl, wr) in [(True, -1, -1), (True, 2, 0), (False, 1, 2)]:
        out, lse = orc.attention(q, k, v, causal=causal, window=(wl, wr), scale=0.5)
        for i in range(Sq):
            lo, hi = _interval(i, Sq, Sk, causal, wl, wr)
            k2, v2 = k.copy(), v.copy()
            sel = np.ones(Sk, bool); sel[lo:hi + 1] = False
            k2[0, sel] = 1e4 * np.sign(_rand(rng, int(sel.sum()), 1, 4))
            v2[0, sel] = -1e4
            o2, l2 = orc.attention(q, k2, v2, causal=causal, window=(wl, wr), scale=0.5)
            assert np.array_equal(o2[0, i], out[0, i]) and np.array_equal(l2[0, :, i], lse[0, :, i])
    # varlen: perturbing sequence 1 leaves sequences 0 and 2 unchanged
    cu = np.array([0, 4, 9, 12], dtype=np.int32)
    qp = _rand(rng, 12, 2, 4); kp = _rand(rng, 12, 1, 4); vp = _rand(rng, 12, 1, 4)
    o1, l1 = orc.attention_varlen(qp, kp, vp, cu, cu, causal=True, scale=0.5)
    kp2, vp2 = kp.copy(), vp.copy(); kp2[4:9] = 1e4; vp2[4:9] = -1e4
    o2, l2 = orc.attention_varlen(qp, kp2, vp2, cu, cu, causal=True, scale=0.5)
    for a, b in ((0, 4), (9, 12)):
        assert np.array_equal(o1[a:b], o2[a:b]) and np.array_equal(l1[:, a:b], l2[:, a:b])
    # decode: rows past the cache length are never read
    qd = _rand(rng, 2, 1, 2, 4); kc = _rand(rng, 2, 8, 1, 4); vc = _rand(rng, 2, 8, 1, 4)
    lens = np.array([5, 8], dtype=np.int32)
    od, ld = orc.attention_decode(qd, kc, vc, lens)
    kc2, vc2 = kc.copy(), vc.copy(); kc2[0, 5:] = 1e4; vc2[0, 5:] = -1e4
    od2, ld2 = orc.attention_decode(qd, kc2, vc2, lens)
    assert np.array_equal(od, od2) and np.array_equal(ld, ld2)


def pin_key_permutation(orc):
    """Without a mask attention treats keys as a set: permuting (k_j, v_j)
    jointly leaves O and LSE unchanged up to rounding."""
    rng = _rng(19)
    q = _rand(rng, 2, 6, 2, 5); k = _rand(rng, 2, 9, 2, 5); v = _rand(rng, 2, 9, 2, 5)
    perm = rng.permutation(9)
    o1, l1 = orc.attention(q, k, v, scale=0.8)
    o2, l2 = orc.attention(q, k[:, perm], v[:, perm], scale=0.8)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13


def pin_gqa_equals_repeated_mha(orc):
    """Hq = G*Hkv equals MHA with each K/V head repeated G times in a row."""
    rng = _rng(20)
    q = _rand(rng, 2, 7, 6, 4); k = _rand(rng, 2, 7, 2, 4); v = _rand(rng, 2, 7, 2, 4)
    o1, l1 = orc.attention(q, k, v, causal=True, scale=0.5)
    o2, l2 = orc.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), causal=True,
                           scale=0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_varlen_equals_per_sequence(orc):
    """Packed sequences equal each sequence run on its own (also with a
    query/key length mismatch and a window)."""
    rng = _rng(21)
    lq = [3, 5, 1, 4]
    lk = [3, 7, 2, 4]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = _rand(rng, cq[-1], 4, 3); k = _rand(rng, ck[-1], 2, 3); v = _rand(rng, ck[-1], 2, 3)
    for (causal, wl, wr) in [(True, -1, -1), (False, -1, -1), (True, 1, 0)]:
        out, lse = orc.attention_varlen(q, k, v, cq, ck, causal=causal, window=(wl, wr),
                                        scale=0.6)
        for z in range(len(lq)):
            o1, l1 = orc.attention(q[None, cq[z]:cq[z + 1]], k[None, ck[z]:ck[z + 1]],
                                   v[None, ck[z]:ck[z + 1]], causal=causal, window=(wl, wr),
                                   scale=0.6)
            assert np.array_equal(out[cq[z]:cq[z + 1]], o1[0])
            assert np.array_equal(lse[:, cq[z]:cq[z + 1]], l1[0])


def pin_decode_equals_last_prefill_row(orc):
    """A one-token decode over a cache of L keys equals the last row of a
    causal prefill over those L keys (and Sq = 1 bottom-right causal)."""
    rng = _rng(22)
    B, cap, Hq, Hkv, d = 3, 11, 4, 2, 5
    lens = np.array([11, 4, 7], dtype=np.int32)
    q = _rand(rng, B, 1, Hq, d); kc = _rand(rng, B, cap, Hkv, d); vc = _rand(rng, B, cap, Hkv, d)
    for (wl, wr) in [(-1, -1), (3, -1)]:
        od, ld = orc.attention_decode(q, kc, vc, lens, causal=True, window=(wl, wr), scale=0.4)
        for b in range(B):
            L = int(lens[b])
            qq = np.concatenate([_rand(rng, 1, L - 1, Hq, d), q[b:b + 1]], axis=1)
            op, lp = orc.attention(qq, kc[b:b + 1, :L], vc[b:b + 1, :L], causal=True,
                                   window=(wl, wr), scale=0.4)
            assert np.array_equal(od[b, 0], op[0, L - 1]) and np.array_equal(ld[b], lp[0, :, L - 1])
            o1, l1 = orc.attention(q[b:b + 1], kc[b:b + 1, :L], vc[b:b + 1, :L], causal=True,
                                   window=(wl, wr), scale=0.4)
            assert np.array_equal(od[b, 0], o1[0, 0]) and np.array_equal(ld[b], l1[0, :, 0])


def pin_key_translation(orc):
    """k_j <- k_j + u for all j: O unchanged, LSE_i shifts by scale*(q_i . u)."""
    rng = _rng(23)
    q = _rand(rng, 1, 6, 2, 4); k = _rand(rng, 1, 8, 1, 4); v = _rand(rng, 1, 8, 1, 4)
    u = _rand(rng, 4)
    for causal in (False, True):
        o1, l1 = orc.attention(q, k, v, causal=causal, scale=0.7)
        o2, l2 = orc.attention(q, k + u, v, causal=causal, scale=0.7)
        shift = 0.7 * np.einsum("bshd,d->bhs", q, u)
        assert np.abs(o1 - o2).max() < 1e-12
        assert np.abs(l2 - l1 - shift).max() < 1e-12


def pin_split_combine(orc):
    """Attention over keys split into chunks, merged with the LSE rule
    (M = max lse_c; LSE = M + ln sum exp(lse_c - M); O = sum exp(lse_c - LSE) O_c),
    equals attention over all keys."""
    rng = _rng(24)
    q = _rand(rng, 5, 6); k = _rand(rng, 23, 6); v = _rand(rng, 23, 6)
    qi = np.arange(5)
    o, l = orc.attention_rows(q, qi, 5, k, v, scale=0.5)
    for cuts in ([0, 8, 16, 23], [0, 1, 23], [0, 11, 12, 20, 23]):
        parts = [orc.attention_rows(q, qi, 5, k[a:b], v[a:b], scale=0.5)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        L = np.stack([p[1] for p in parts])           # [C, n]
        M = L.max(0)
        lse = M + np.log(np.exp(L - M).sum(0))
        out = sum(np.exp(p[1] - lse)[:, None] * p[0] for p in parts)
        assert np.abs(lse - l).max() < 1e-12 and np.abs(out - o).max() < 1e-12


def pin_fully_masked_rows(orc):
    """Sq > Sk with bottom-right causal: the first Sq - Sk rows see no key, so
    O = 0 and LSE = -inf; later rows are finite."""
    rng = _rng(25)
    q = _rand(rng, 1, 6, 1, 3); k = _rand(rng, 1, 4, 1, 3); v = _rand(rng, 1, 4, 1, 3)
    out, lse = orc.attention(q, k, v, causal=True, scale=1.0)
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    lens = np.array([0, 3], dtype=np.int32)
    od, ld = orc.attention_decode(q[:, :1].repeat(2, 0), np.concatenate([k, k]),
                                  np.concatenate([v, v]), lens)
    assert np.all(od[0] == 0) and np.isneginf(ld[0, 0]) and np.isfinite(ld[1, 0])


def pin_large_scores_stable(orc):
    """Scores of several hundred: exponentials are taken relative to the row
    maximum (as in the page's worked example), so nothing overflows. With
    scores 0, 100, ..., 900 the weight sits on the last key to within e^-100."""
    n, d = 10, 4
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1000.0
    k = np.zeros((1, n, 1, d)); k[0, :, 0, 0] = np.arange(n) / 10.0
    v = _rand(_rng(27), 1, n, 1, d)
    for causal in (False, True):
        out, lse = orc.attention(q, k, v, causal=causal, scale=1.0)
        assert np.all(np.isfinite(out)) and np.isfinite(lse).all()
        assert abs(lse[0, 0, 0] - 900.0) < 1e-12
        assert np.abs(out[0, 0, 0] - v[0, n - 1, 0]).max() < 1e-12


def pin_mpmath_brute_force(orc):
    """30-digit brute force (fully materialised scores, weights and output)
    on tiny inputs, every mask mode, GQA."""
    import mpmath
    mpmath.mp.dps = 30
    rng = _rng(26)
    B, Hq, Hkv, d = 1, 4, 2, 3
    for (Sq, Sk, causal, wl, wr) in [(5, 5, False, -1, -1), (5, 5, True, -1, -1),
                                     (3, 6, True, -1, -1), (6, 6, True, 2, 0),
                                     (6, 6, False, 1, 2)]:
        q = _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
        scale = 0.77
        out, lse = orc.attention(q, k, v, causal=causal, window=(wl, wr), scale=scale)
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                pos = i + Sk - Sq
                keys = [j for j in range(Sk)
                        if (not causal or j <= pos) and (wl < 0 or j >= pos - wl)
                        and (wr < 0 or j <= pos + wr)]
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, i, h, t]) * mpmath.mpf(k[0, j, g, t])
                                                     for t in range(d)) for j in keys]
                e = [mpmath.exp(x) for x in s]
                z = mpmath.fsum(e)
                assert abs(float(mpmath.log(z)) - lse[0, h, i]) < 1e-12
                for t in range(d):
                    o = mpmath.fsum(ej * mpmath.mpf(v[0, j, g, t]) for ej, j in zip(e, keys)) / z
                    assert abs(float(o) - out[0, i, h, t]) < 1e-12


# ---------------------------------------------------------------------------
# Gradients (fa_oracle_bwd).  The pages fix only what the backward computes
# (the gradients of the forward definition); these pins tie the oracle's
# chain rule to the forward oracle (finite differences), to torch autograd,
# and to exact identities of softmax attention.

_BWD_CASES = [(4, 4, False, -1, -1), (4, 4, True, -1, -1), (3, 6, True, -1, -1),
              (6, 6, True, 2, 0), (5, 5, False, 1, 2), (6, 3, True, -1, -1)]


def pin_bwd_finite_differences(orc):
    """dq, dk, dv equal central differences of L = sum(dout * O) through the
    forward oracle, element by element (GQA, every mask mode, rows with no
    visible key)."""
    rng = _rng(40)
    B, Hq, Hkv, d, scale, h = 1, 2, 1, 3, 0.83, 1e-6
    for (Sq, Sk, causal, wl, wr) in _BWD_CASES:
        q = _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
        go = _rand(rng, B, Sq, Hq, d)
        dq, dk, dv = orc.attention_bwd(q, k, v, go, causal=causal, window=(wl, wr), scale=scale)

        def loss(qq, kk, vv):
            o, _ = orc.attention(qq, kk, vv, causal=causal, window=(wl, wr), scale=scale)
            return float((o * go).sum())

        for x, gx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = [q, k, v]; args_p[which] = xp
                args_m = [q, k, v]; args_m[which] = xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert np.abs(num - gx).max() < 1e-7 * max(1.0, np.abs(gx).max()), (Sq, Sk, causal, which)


def _torch_grads(q, k, v, go, causal, wl, wr, scale):
    """float64 autograd through an explicit masked softmax (GQA by repeating
    K/V heads, rows with no visible key give zero weights)."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).clone().requires_grad_(True)
    G = tq.shape[1] // tk.shape[1]
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    mask = _visible_band(q.shape[1], k.shape[1], causal, wl, wr)
    s = (tq @ kk.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    m = s.amax(-1, keepdim=True).clamp_min(-1e300)      # rows with no key: all -inf
    e = torch.exp(s - m).masked_fill(~mask, 0.0)
    z = e.sum(-1, keepdim=True)
    p = e / torch.where(z > 0, z, torch.ones_like(z))
    o = p @ vv
    o.backward(torch.from_numpy(go).permute(0, 2, 1, 3))
    return (tq.grad.permute(0, 2, 1, 3).numpy(), tk.grad.permute(0, 2, 1, 3).numpy(),
            tv.grad.permute(0, 2, 1, 3).numpy())


def pin_bwd_torch_autograd(orc):
    """torch float64 autograd of the same attention (independent code path)."""
    rng = _rng(41)
    B, Hq, Hkv, d, scale = 2, 4, 2, 8, 0.35
    for (Sq, Sk, causal, wl, wr) in _BWD_CASES + [(17, 23, True, 5, -1), (23, 17, False, -1, -1)]:
        q = _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
        go = _rand(rng, B, Sq, Hq, d)
        got = orc.attention_bwd(q, k, v, go, causal=causal, window=(wl, wr), scale=scale)
        ref = _torch_grads(q, k, v, go, causal, wl, wr, scale)
        for a, r in zip(got, ref):
            assert np.abs(a - r).max() < 1e-12, (Sq, Sk, causal, wl, wr)


def pin_bwd_identities(orc):
    """Exact identities: the weights of a row sum to one, so sum_j dV_j =
    sum of dout over rows with a visible key; adding one vector to every key
    leaves O unchanged, so sum_j dK_j = 0; a key no row sees gets dK = dV = 0;
    a row with no visible key gets dQ = 0."""
    rng = _rng(42)
    B, Hq, Hkv, d = 2, 4, 2, 5
    for (Sq, Sk, causal, wl, wr) in _BWD_CASES:
        q = _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
        go = _rand(rng, B, Sq, Hq, d)
        dq, dk, dv = orc.attention_bwd(q, k, v, go, causal=causal, window=(wl, wr), scale=0.6)
        vis = _visible_band(Sq, Sk, causal, wl, wr).numpy()
        rows = vis.any(1)
        G = Hq // Hkv
        for g in range(Hkv):
            want = go[:, rows][:, :, g * G:(g + 1) * G].sum(axis=(1, 2))
            assert np.abs(dv[:, :, g].sum(1) - want).max() < 1e-12
            assert np.abs(dk[:, :, g].sum(1)).max() < 1e-12
        assert np.all(dq[:, ~rows] == 0)
        cols = vis.any(0)
        assert np.all(dk[:, ~cols] == 0) and np.all(dv[:, ~cols] == 0)


def pin_bwd_gqa_equals_repeated_mha(orc):
    """GQA gradients equal MHA gradients with K/V heads repeated, dK/dV summed
    over each group."""
    rng = _rng(43)
    B, Sq, Sk, Hq, Hkv, d = 1, 7, 9, 6, 2, 4
    q = _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
    go = _rand(rng, B, Sq, Hq, d)
    G = Hq // Hkv
    dq, dk, dv = orc.attention_bwd(q, k, v, go, causal=True, scale=0.5)
    dq2, dk2, dv2 = orc.attention_bwd(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), go,
                                      causal=True, scale=0.5)
    assert np.abs(dq - dq2).max() < 1e-12
    assert np.abs(dk - dk2.reshape(B, Sk, Hkv, G, d).sum(3)).max() < 1e-12
    assert np.abs(dv - dv2.reshape(B, Sk, Hkv, G, d).sum(3)).max() < 1e-12


def _paginate(rng, cache, lens, page_size, spare_pages=2):
    """Scatter a contiguous cache [B, cap, Hkv, d] into a shuffled page pool
    (each sequence's first ceil(len/page_size) pages, in random physical
    order, plus unreferenced spare pages of random data).  Pages are cut by
    reshaping each sequence's rows; table entries past a sequence's pages
    hold an index outside the pool, so reading one is an error.
    -> (pages [num_pages, page_size, Hkv, d], block_table [B, max_pages])."""
    B, cap, Hkv, d = cache.shape
    assert cap % page_size == 0
    need = [-(-int(n) // page_size) for n in lens]
    max_pages = max(max(need), 1)
    num_pages = sum(need) + spare_pages
    perm = rng.permutation(num_pages)
    pages = _rand(rng, num_pages, page_size, Hkv, d)
    table = np.full((B, max_pages), num_pages + 7, dtype=np.int32)
    nxt = 0
    for b in range(B):
        chunks = cache[b].reshape(cap // page_size, page_size, Hkv, d)
        for pg in range(need[b]):
            pages[perm[nxt]] = chunks[pg]
            table[b, pg] = perm[nxt]
            nxt += 1
    return pages, table


def pin_paged_equals_contiguous(orc):
    """A paged cache (shuffled pages, garbage in unused rows and spare pages)
    gives exactly the contiguous-cache decode of the same keys."""
    rng = _rng(60)
    B, Hq, Hkv, d = 3, 4, 2, 5
    for page_size, lens in [(1, [3, 0, 5]), (3, [9, 4, 1]), (4, [8, 7, 12]), (8, [16, 1, 9])]:
        cap = page_size * -(-max(lens) // page_size)
        lens = np.array(lens, dtype=np.int32)
        q = _rand(rng, B, 1, Hq, d)
        kc = _rand(rng, B, cap, Hkv, d); vc = _rand(rng, B, cap, Hkv, d)
        pk, table = _paginate(np.random.default_rng(page_size), kc, lens, page_size)
        pv, table_v = _paginate(np.random.default_rng(page_size), vc, lens, page_size)
        assert np.array_equal(table, table_v)
        for (wl, wr) in [(-1, -1), (2, -1)]:
            o1, l1, pk2, pv2 = orc.attention_decode_paged(q, pk, pv, table, lens, causal=True,
                                                          window=(wl, wr), scale=0.6)
            o2, l2 = orc.attention_decode(q, kc, vc, lens, causal=True, window=(wl, wr), scale=0.6)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), (page_size, wl)
            assert np.array_equal(pk2, pk) and np.array_equal(pv2, pv)   # nothing appended


def pin_paged_append(orc):
    """Appending writes the new key/value row at position cache_seqlens[b]
    of its sequence (and nowhere else), and the query then sees that row:
    the result equals the contiguous decode over the cache with the row in
    place and one more key."""
    rng = _rng(61)
    B, Hq, Hkv, d, page_size = 3, 6, 2, 4, 4
    lens = np.array([0, 7, 8], dtype=np.int32)            # empty, mid-page, page boundary
    cap = 12
    q = _rand(rng, B, 1, Hq, d)
    kc = _rand(rng, B, cap, Hkv, d); vc = _rand(rng, B, cap, Hkv, d)
    kn = _rand(rng, B, 1, Hkv, d); vn = _rand(rng, B, 1, Hkv, d)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b, lens[b]] = kn[b, 0]
        vc2[b, lens[b]] = vn[b, 0]
    # pages hold the old contents (row lens[b] is stale) for len+1 rows
    pk, table = _paginate(np.random.default_rng(5), kc, lens + 1, page_size)
    pv, _ = _paginate(np.random.default_rng(5), vc, lens + 1, page_size)
    pk_want, _ = _paginate(np.random.default_rng(5), kc2, lens + 1, page_size)
    pv_want, _ = _paginate(np.random.default_rng(5), vc2, lens + 1, page_size)
    for (wl, wr) in [(-1, -1), (3, -1)]:
        o1, l1, pk2, pv2 = orc.attention_decode_paged(q, pk, pv, table, lens, kn, vn, causal=True,
                                                      window=(wl, wr), scale=0.45)
        o2, l2 = orc.attention_decode(q, kc2, vc2, lens + 1, causal=True, window=(wl, wr),
                                      scale=0.45)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), wl
        assert np.array_equal(pk2, pk_want) and np.array_equal(pv2, pv_want)


def pin_paged_append_zero_query(orc):
    """Q = 0 with an append: LSE = ln(cache_seqlens + 1) and O is the mean
    of the cached V rows and the new one."""
    rng = _rng(62)
    B, Hq, Hkv, d, page_size = 2, 2, 1, 3, 2
    lens = np.array([4, 1], dtype=np.int32)
    kc = _rand(rng, B, 6, Hkv, d); vc = _rand(rng, B, 6, Hkv, d)
    kn = _rand(rng, B, 1, Hkv, d); vn = _rand(rng, B, 1, Hkv, d)
    pk, table = _paginate(np.random.default_rng(9), kc, lens + 1, page_size)
    pv, _ = _paginate(np.random.default_rng(9), vc, lens + 1, page_size)
    out, lse, _, _ = orc.attention_decode_paged(np.zeros((B, 1, Hq, d)), pk, pv, table, lens,
                                                kn, vn)
    for b in range(B):
        L = int(lens[b])
        mean = (vc[b, :L, 0].sum(0) + vn[b, 0, 0]) / (L + 1)
        for h in range(Hq):
            assert abs(lse[b, h] - math.log(L + 1)) < 1e-13
            assert np.abs(out[b, 0, h] - mean).max() < 1e-13


_MOD_CASES = [  # Sq, Sk, causal, wl, wr, softcap, with ALiBi
    (6, 6, False, -1, -1, 0.0, True), (6, 6, True, -1, -1, 0.0, True), (5, 9, True, -1, -1, 0.0, True),
    (9, 5, False, 2, 1, 0.0, True), (6, 6, True, -1, -1, 1.5, False), (7, 7, False, -1, -1, 2.0, False),
    (8, 8, True, 3, -1, 1.2, True), (4, 10, False, -1, -1, 0.7, True),
]


def _mod_reference(q, k, v, causal, wl, wr, scale, softcap, slopes):
    """torch float64: scores, soft-capping, ALiBi bias from explicit
    positions, mask, softmax, logsumexp, all written out independently."""
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    s = scale * torch.matmul(qt, kt.transpose(-1, -2))
    if softcap > 0:
        s = softcap * torch.tanh(s / softcap)
    if slopes is not None:
        qpos = torch.arange(Sq, dtype=torch.float64)[:, None] + (Sk - Sq)
        kpos = torch.arange(Sk, dtype=torch.float64)[None, :]
        s = s - torch.from_numpy(slopes)[:, None, None] * (qpos - kpos).abs()
    vis = _visible_band(Sq, Sk, causal, wl, wr)
    s = s.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    w = torch.softmax(s, dim=-1).nan_to_num(0.0)
    o = torch.matmul(w, vt).permute(0, 2, 1, 3)
    return o.numpy(), lse.numpy()


def pin_mod_torch_reference(orc):
    """Soft-capping and ALiBi against an independent torch float64 version
    (every mask mode, Sq != Sk alignment, GQA)."""
    rng = _rng(70)
    B, Hq, Hkv, d, scale = 2, 4, 2, 6, 0.8
    for (Sq, Sk, causal, wl, wr, cap, alibi) in _MOD_CASES:
        q = 2 * _rand(rng, B, Sq, Hq, d); k = _rand(rng, B, Sk, Hkv, d); v = _rand(rng, B, Sk, Hkv, d)
        slopes = np.array([0.5, 0.25, 0.125, 0.0625]) if alibi else None
        o1, l1 = orc.attention_mod(q, k, v, causal=causal, window=(wl, wr), scale=scale,
                                   softcap=cap, alibi_slopes=slopes)
        o2, l2 = _mod_reference(q, k, v, causal, wl, wr, scale, cap, slopes)
        fin = np.isfinite(l2)
        assert np.array_equal(np.isfinite(l1), fin)
        assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1[fin] - l2[fin]).max() < 1e-12


def pin_mod_neutral(orc):
    """No cap and zero (or no) slopes give the plain definition exactly."""
    rng = _rng(71)
    q = _rand(rng, 1, 7, 4, 5); k = _rand(rng, 1, 9, 2, 5); v = _rand(rng, 1, 9, 2, 5)
    for causal in (False, True):
        o0, l0 = orc.attention(q, k, v, causal=causal, scale=0.6)
        for slopes in (None, np.zeros(4)):
            o1, l1 = orc.attention_mod(q, k, v, causal=causal, scale=0.6, alibi_slopes=slopes)
            assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def pin_alibi_zero_query_closed_form(orc):
    """Q = 0: scores are -slope * distance, so LSE_i is the log of a sum of
    two geometric series (keys at or before the row, keys after it)."""
    n, slope = 9, 0.3
    rng = _rng(72)
    k = _rand(rng, 1, n, 1, 4); v = _rand(rng, 1, n, 1, 4)
    r = math.exp(-slope)
    for causal in (True, False):
        _, lse = orc.attention_mod(np.zeros((1, n, 1, 4)), k, v, causal=causal,
                                   alibi_slopes=np.array([slope]))
        for i in range(n):
            before = (1 - r ** (i + 1)) / (1 - r)
            after = 0.0 if causal else r * (1 - r ** (n - 1 - i)) / (1 - r)
            assert abs(lse[0, 0, i] - math.log(before + after)) < 1e-13


def pin_softcap_saturates(orc):
    """Scores of +-1e6 capped at 5 become +-5: two keys give weights
    e^5 / (e^5 + e^-5) and LSE = ln(e^5 + e^-5); a huge cap is the plain
    definition."""
    d = 2
    q = np.array([[[[1000.0, 0.0]]]])
    k = np.array([[[[1000.0, 0.0]], [[-1000.0, 0.0]]]])
    v = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    o, lse = orc.attention_mod(q, k, v, scale=1.0, softcap=5.0)
    w = math.exp(5) / (math.exp(5) + math.exp(-5))
    assert abs(lse[0, 0, 0] - math.log(math.exp(5) + math.exp(-5))) < 1e-13
    assert abs(o[0, 0, 0, 0] - w) < 1e-13 and abs(o[0, 0, 0, 1] - (1 - w)) < 1e-13
    rng = _rng(73)
    q = _rand(rng, 1, 5, 2, d); k = _rand(rng, 1, 6, 2, d); v = _rand(rng, 1, 6, 2, d)
    o0, l0 = orc.attention(q, k, v, causal=True, scale=0.5)
    o1, l1 = orc.attention_mod(q, k, v, causal=True, scale=0.5, softcap=1e7)
    assert np.abs(o0 - o1).max() < 1e-10 and np.abs(l0 - l1).max() < 1e-10


def pin_e4m3_decoder(orc):
    """Every one of the 256 e4m3 codes decodes to torch's float8_e4m3fn value
    (a library routine of the same format), NaN exactly at the two NaN codes;
    spot values from the format: 0x38 = 1, 0x7e = 448 (the largest), 0x08 =
    2^-6 (the smallest normal), 0x01 = 2^-9 (the smallest subnormal)."""
    import oracle as _o
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = _o.decode_e4m3(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and int(nan.sum()) == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0xB8] == -1.0 and got[0x80] == 0.0


def pin_fp8_attention(orc):
    """The 8-bit entry of the oracle is the plain definition on descaled
    values: equal to attention() on torch-decoded inputs times the scales;
    all-zero query codes give LSE = ln(#visible)."""
    rng = _rng(80)
    B, Sq, Sk, Hq, Hkv, d = 1, 6, 9, 4, 2, 8
    mk = lambda *sh: torch.from_numpy(rng.integers(0, 256, size=sh).astype(np.uint8))
    q8, k8, v8 = mk(B, Sq, Hq, d), mk(B, Sk, Hkv, d), mk(B, Sk, Hkv, d)
    for t in (q8, k8, v8):                     # no NaN codes
        t[(t & 0x7F) == 0x7F] = 0x38
    dq, dk, dv = 0.01, 0.02, 0.5
    dec = lambda t, s: t.view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    for causal in (False, True):
        o1, l1 = orc.attention_fp8(q8, k8, v8, dq, dk, dv, causal=causal, scale=0.3)
        o2, l2 = orc.attention(dec(q8, dq), dec(k8, dk), dec(v8, dv), causal=causal, scale=0.3)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    _, lz = orc.attention_fp8(torch.zeros_like(q8), k8, v8, dq, dk, dv, causal=True)
    for i in range(Sq):
        assert abs(lz[0, 0, i] - math.log(i + Sk - Sq + 1)) < 1e-13


# -- the row-sampled entry (used by the full-size GPU checks) ----------------
_ROW_CASES = [  # Sq, Sk, causal, wl, wr: every mask mode the sampled checks use
    (40, 40, False, -1, -1), (40, 40, True, -1, -1), (40, 40, True, 7, -1),
    (40, 40, True, 7, 7), (40, 40, False, 5, 9), (25, 40, True, -1, -1),
    (40, 25, True, -1, -1), (30, 45, True, 6, 0), (45, 30, False, 4, 2),
]


def _unsorted_rows(rng, Sq):
    """Row indices in no particular order: both ends, a repeat and random rows."""
    qi = np.concatenate([[Sq - 1, 0], rng.integers(0, Sq, 9), [Sq // 2, Sq // 2]])
    return rng.permutation(qi)


def pin_rows_match_sdpa_masked(orc):
    """attention_rows on unsorted row indices equals torch float64 SDPA (mask
    built from torch band helpers) row by row, in every mask mode and with
    Sq < Sk and Sq > Sk (bottom-right alignment)."""
    rng = _rng(31)
    for (Sq, Sk, causal, wl, wr) in _ROW_CASES:
        d = 5
        q = _rand(rng, 1, Sq, 1, d); k = _rand(rng, 1, Sk, 1, d); v = _rand(rng, 1, Sk, 1, d)
        ro, rl = _sdpa_reference(q, k, v, causal, wl, wr, 0.6)
        qi = _unsorted_rows(rng, Sq)
        o, l = orc.attention_rows(q[0, qi, 0], qi, Sq, k[0, :, 0], v[0, :, 0], causal=causal,
                                  window=(wl, wr), scale=0.6)
        for r, i in enumerate(qi):
            if np.isneginf(rl[0, 0, i]):          # no visible key: O = 0, LSE = -inf
                assert np.isneginf(l[r]) and np.all(o[r] == 0.0), (Sq, Sk, causal, wl, wr, i)
                continue
            assert abs(l[r] - rl[0, 0, i]) < 1e-12, (Sq, Sk, causal, wl, wr, i)
            assert np.abs(o[r] - ro[0, i, 0]).max() < 1e-12, (Sq, Sk, causal, wl, wr, i)


def pin_rows_zero_query_closed_form(orc):
    """attention_rows with Q = 0: LSE of sampled row i = ln(#visible keys of
    row i), O = mean of those value rows; includes the decode form (one
    query at the last position of its cache) and unsorted indices."""
    rng = _rng(32)
    cases = _ROW_CASES + [(1, 37, True, -1, -1), (1, 37, False, 10, -1)]
    for (Sq, Sk, causal, wl, wr) in cases:
        d = 4
        k = _rand(rng, Sk, d); v = _rand(rng, Sk, d)
        qi = _unsorted_rows(rng, Sq)
        o, l = orc.attention_rows(np.zeros((len(qi), d)), qi, Sq, k, v, causal=causal,
                                  window=(wl, wr), scale=1.3)
        for r, i in enumerate(qi):
            lo, hi = _interval(int(i), Sq, Sk, causal, wl, wr)
            lo = max(lo, 0)
            if hi < lo:
                assert np.isneginf(l[r]) and np.all(o[r] == 0.0)
                continue
            assert abs(l[r] - math.log(hi - lo + 1)) < 1e-13, (Sq, Sk, causal, wl, wr, i)
            assert np.abs(o[r] - v[lo:hi + 1].mean(0)).max() < 1e-13


PINS = [
    pin_worked_example, pin_torch_sdpa, pin_zero_query_closed_form, pin_varlen_zero_query,
    pin_decode_zero_query, pin_constant_v, pin_single_visible_key, pin_one_hot_values,
    pin_masked_keys_no_effect, pin_key_permutation, pin_gqa_equals_repeated_mha,
    pin_varlen_equals_per_sequence, pin_decode_equals_last_prefill_row, pin_key_translation,
    pin_split_combine, pin_fully_masked_rows, pin_large_scores_stable, pin_mpmath_brute_force,
    pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_identities,
    pin_bwd_gqa_equals_repeated_mha, pin_paged_equals_contiguous, pin_paged_append,
    pin_paged_append_zero_query, pin_mod_torch_reference, pin_mod_neutral,
    pin_alibi_zero_query_closed_form, pin_softcap_saturates, pin_e4m3_decoder, pin_fp8_attention,
    pin_rows_match_sdpa_masked, pin_rows_zero_query_closed_form,
]
