"""Parity checks of GPU results against the fp64 oracle -- test
infrastructure only (used by tests/ and __graft_entry__.smoke()).

Forward (``compare``): no attention arithmetic here, only the comparison.

Tolerances (stated for the attention path): max |dO| <= 1e-2 for bf16/fp16
outputs and max |dLSE| <= 1e-3, both against the unrounded fp64 oracle.

A correctly rounded bf16 output can itself be up to half a bf16 ulp away
from the exact value, i.e. 1/64 = 0.0156 when |O| is in [4, 8).  Rows that
see only a handful of keys can reach such magnitudes with N(0,1) values.
So an element whose error exceeds 1e-2 is accepted only when the exact
value is that large AND the GPU value is within one output ulp of it (at
most one rounding step away); every such element is counted and reported,
never hidden.
"""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 1e-2
LSE_TOL = 1e-3
OUT_TYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output format at |x| (bf16: 8 significand bits, fp16: 11)."""
    mant = 8 if dtype == "bf16" else 11
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - (mant - 1))


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, label: str = "") -> dict:
    """Assert parity; return the statistics (max errors, counts)."""
    og, orf = to_f64(o_gpu), to_f64(o_ref)
    lg, lr = to_f64(lse_gpu), to_f64(lse_ref)
    assert og.shape == orf.shape, (og.shape, orf.shape)
    assert lg.shape == lr.shape, (lg.shape, lr.shape)
    assert np.isfinite(og).all(), f"{label}: non-finite output"
    err = np.abs(og - orf)
    over = err > O_TOL
    n_over = int(over.sum())
    if n_over:
        within_ulp = err[over] <= ulp(orf[over], dtype) * (1 + 1e-9)
        big = np.abs(orf[over]) >= 2.0
        assert within_ulp.all() and big.all(), (
            f"{label}: {n_over} outputs exceed {O_TOL}; worst err {err.max():.4g} at "
            f"|O_ref|={np.abs(orf.reshape(-1)[err.argmax()]):.4g}")
    # LSE: -inf exactly where the oracle has no visible key
    ninf_ref = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), ninf_ref), f"{label}: -inf LSE pattern differs"
    fin = ~ninf_ref
    lse_err = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
    assert lse_err <= LSE_TOL, f"{label}: max |dLSE| {lse_err:.3g} > {LSE_TOL}"
    # the rounding floor of the output format (the exact value rounded once)
    # and the largest distance of a GPU value from that rounded value
    rounded = to_f64(torch.from_numpy(orf).to(OUT_TYPES[dtype]))
    floor = float(np.abs(rounded - orf).max()) if err.size else 0.0
    excess = float(np.abs(og - rounded).max()) if err.size else 0.0
    return {"max_dO": float(err.max()) if err.size else 0.0, "n_over_1e-2": n_over,
            "max_dLSE": lse_err, "floor_dO": floor, "excess_dO": excess, "n": int(err.size)}


def merge(stats: list) -> dict:
    """Combine the statistics of several compare() calls."""
    return {"max_dO": max(s["max_dO"] for s in stats),
            "n_over_1e-2": sum(s["n_over_1e-2"] for s in stats),
            "max_dLSE": max(s["max_dLSE"] for s in stats),
            "floor_dO": max(s["floor_dO"] for s in stats),
            "excess_dO": max(s["excess_dO"] for s in stats),
            "n": sum(s["n"] for s in stats)}


def log(stats: dict, label: str) -> None:
    print(f"[parity] {label}: " + ", ".join(f"{k}={v:.4g}" if isinstance(v, float)
                                           else f"{k}={v}" for k, v in stats.items()),
          flush=True)


# -- backward ------------------------------------------------------------------
def _band(Sq, Sk, causal, wl, wr):
    """Boolean [Sq,Sk] visibility from band helpers: query i sits at key
    position i + Sk - Sq; inclusive window bounds, -1 unbounded."""
    delta = Sk - Sq
    m = np.ones((Sq, Sk), dtype=bool)
    if causal:
        m &= np.tril(np.ones((Sq, Sk), dtype=bool), k=delta)
    if wr >= 0:
        m &= np.tril(np.ones((Sq, Sk), dtype=bool), k=delta + wr)
    if wl >= 0:
        m &= np.triu(np.ones((Sq, Sk), dtype=bool), k=delta - wl)
    return m


def grad_error_bounds(q, k, v, go, causal, window, scale):
    """Per-element error bounds of the three gradients (tolerances only; the
    expected values come from the oracle).

    Each gradient element is a sum over rows or keys:
        dV_jc = sum_i P_ij dO_ic,   dK_jc = scale sum_i dS_ij Q_ic,
        dQ_ic = scale sum_j dS_ij K_jc,   dS_ij = P_ij (dP_ij - D_i),
    and the kernels round P and dS to the input dtype before these products
    (relative error <= 2^-9 per term; 2^-12 for fp16).  Under cancellation
    the error is relative to the sum of the absolute terms A, not to the
    result, so the bound is 2^-8 * A (a 2x margin), A summed here in fp64
    with P, dP and dS written out per head.
    The row term D_i = dO_i . O_i is formed from the forward's 16-bit output,
    so each dS_ij of row i carries an error dD_i <= E_i =
    2^-7 sum_c |dO_ic| (|O_ic| + 2^-7) (output rounding 2^-9 |O| plus the
    forward's own error); it adds scale E_i |sum_j P_ij K_jc| to dQ and
    scale sum_i P_ij E_i |Q_ic| to dK.  The final rounding of each gradient
    to the input dtype adds 2^-8 |g| (in ``check_grad``)."""
    sc = scale if scale is not None else q.shape[-1] ** -0.5
    qf, kf, vf, gf = (x.double().numpy() for x in (q, k, v, go))
    B, Sq, Hq, d = qf.shape
    Sk, Hkv = kf.shape[1], kf.shape[2]
    G = Hq // Hkv
    vis = _band(Sq, Sk, causal, window[0], window[1])
    bq, bk, bv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = np.where(vis, sc * qf[b, :, h] @ kf[b, :, g].T, -np.inf)
            m = s.max(1, keepdims=True)
            m[~np.isfinite(m)] = 0.0
            e = np.where(vis, np.exp(s - m), 0.0)
            z = e.sum(1, keepdims=True)
            P = e / np.where(z > 0, z, 1.0)
            dO = gf[b, :, h]
            O = P @ vf[b, :, g]
            dP = dO @ vf[b, :, g].T
            D = (dO * O).sum(1, keepdims=True)
            aS = np.abs(P * (dP - D))
            E = 2.0 ** -7 * (np.abs(dO) * (np.abs(O) + 2.0 ** -7)).sum(1, keepdims=True)
            bv[b, :, g] += 2.0 ** -8 * (P.T @ np.abs(dO))
            bk[b, :, g] += abs(sc) * (2.0 ** -8 * (aS.T @ np.abs(qf[b, :, h])) + P.T @ (E * np.abs(qf[b, :, h])))
            bq[b, :, h] = abs(sc) * (2.0 ** -8 * (aS @ np.abs(kf[b, :, g])) + E * np.abs(P @ kf[b, :, g]))
    return bq, bk, bv


def check_grad(name, got, ref, extra):
    """Assert |got - ref| <= 2^-8 |ref| + extra element by element; print the worst ratio."""
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite gradient"
    err = np.abs(g - ref)
    tol = 2.0 ** -8 * np.abs(ref) + extra
    bad = err > tol
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if ref.size:
        w = int(np.argmax(err / np.maximum(tol, 1e-300)))
        worst = float(err.reshape(-1)[w] / max(tol.reshape(-1)[w], 1e-300))
        print(f"[grad] {name}: max|err| {err.max():.3e}  rms(ref) {rms:.3e}  worst err/tol "
              f"{worst:.3f} at ref {ref.reshape(-1)[w]:.4e} got {g.reshape(-1)[w]:.4e} "
              f"(index {np.unravel_index(w, ref.shape)})", flush=True)
    assert not bad.any(), f"{name}: {int(bad.sum())} elements exceed the tolerance"
