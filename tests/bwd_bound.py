"""Per-element error bound for the backward kernels' gradients (test helper).

The kernels compute the gradients of attention over a key set with bf16 operands and float32
accumulation (see the backward's readings):
  P = exp(scale Q K^T - LSE) on the key set (float32, from the forward's LSE),
  dP = dO V^T                                (bf16 inputs, float32 sums of D = 128 terms),
  Dr = sum_d dO[r, d] O[r, d]                (O as the forward handed it over, float32 sum),
  dS = P (dP - Dr)   [times 1 - tanh^2 with a softcap],
  dV = P_b^T dO,  dQ = scale dS_b K,  dK = scale dS_b^T Q,
where P_b and dS_b are P and dS rounded to bf16 for the MFMA products.

With u = 2^-8 the bf16 unit roundoff and eps = 2^-24 that of float32, each gradient entry is a
sum of n products whose rounding errors add up to at most
  dV[k, d]: (u + n eps) * sum_r |P[r, k]| |dO[r, d]|
  dQ[r, d]: scale * ((2u + n eps) * sum_k A[r, k] |K[k, d]| + dD_r * sum_k |P g|[r, k] |K[k, d]|)
  dK[k, d]: scale * ((2u + n eps) * sum_r A[r, k] |Q[r, d]| + sum_r |P g|[r, k] dD_r |Q[r, d]|)
with g the softcap factor (1 without one), A = |P| g (|dP - Dr| + D eps |dO| |V|^T) the size of
dS including the float32 error of dP (2u: one u for dS's rounding to bf16, one as margin, since
both kernels now form dS from the float32 P), and dD_r the error of Dr:
|sum_d dO (O_used - O)| (O_used the O the kernels were given, O the exact one) plus its float32
rounding.  n is the number of products summed into the entry (keys of the row for dQ, rows that
see the key for dK and dV), so the bound grows with the worst-case accumulation; the recomputed
P also carries the float32 error of the forward's LSE and of exp (a relative 1e-5 is added to u).
Summed over the query heads of a kv head for dK and dV, like the gradients.  Everything here is
float64 NumPy, computed from the same inputs as the oracle but not by it.
"""
from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -8 + 1e-5
EPS32 = 2.0 ** -24


def _head(q, k, v, do, mask, scale, o_used, softcap):
    x = scale * (q @ k.T)
    g = np.ones_like(x)
    if softcap > 0.0:
        t = np.tanh(x / softcap)
        x = softcap * t
        g = 1.0 - t * t
    s = np.where(mask, x, -np.inf)
    m = s.max(axis=1, keepdims=True) if s.shape[1] else np.full((s.shape[0], 1), -np.inf)
    empty = np.isneginf(m)
    p = np.exp(s - np.where(empty, 0.0, m))
    p = np.where(empty, 0.0, p / np.where(empty, 1.0, p.sum(axis=1, keepdims=True)))
    o = p @ v
    dp = do @ v.T
    D = q.shape[1]
    d_exact = (do * o).sum(axis=1, keepdims=True)
    d_used = (do * o_used).sum(axis=1, keepdims=True)
    dd = np.abs(d_used - d_exact) + D * EPS32 * (np.abs(do) * np.abs(o_used)).sum(axis=1, keepdims=True)
    pg = p * g
    a = pg * (np.abs(dp - d_exact) + D * EPS32 * (np.abs(do) @ np.abs(v).T))
    n_row = mask.sum(axis=1, keepdims=True)            # products per dQ entry
    n_col = mask.sum(axis=0)[:, None]                  # products per dK / dV entry (this head)
    bq = scale * ((2 * U + n_row * EPS32) * (a @ np.abs(k)) + dd * (pg @ np.abs(k)))
    bk = scale * ((2 * U + n_col * EPS32) * (a.T @ np.abs(q)) + (pg * dd).T @ np.abs(q))
    bv = (U + n_col * EPS32) * (p.T @ np.abs(do))
    return bq, bk, bv


def grad_bounds(q, k, v, do, o_used, mask_of, scale=None, softcap=0.0):
    """Bounds [B,Sq,Hq,D], [B,Sk,Hkv,D], [B,Sk,Hkv,D] for dQ, dK, dV.  q/k/v/do/o_used are float64
    (or bf16 bits widened by the caller); mask_of(b, h) gives the [Sq, Sk] key set of query head h."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    G = Hq // Hkv
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            x, y, z = _head(q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h], mask_of(b, h), scale, o_used[b, :, h],
                            softcap)
            bq[b, :, h] = x
            bk[b, :, hk] += y
            bv[b, :, hk] += z
    return bq, bk, bv


def check_within(name, got, ref, bound):
    """|got - ref| <= 2 * bound + 1e-6 everywhere (the bound is a worst case; the factor 2 covers
    the terms it rounds, e.g. the float32 exp and the LSE)."""
    err = np.abs(got - ref)
    ok = err <= 2.0 * bound + 1e-6
    assert np.isfinite(got).all(), f"{name}: non-finite gradient"
    if not ok.all():
        i = np.unravel_index(np.argmax(err - 2.0 * bound), err.shape)
        raise AssertionError(f"{name}: error {err[i]:.3e} above 2 x bound {bound[i]:.3e} at {i}")
    ratio = float((err / (2.0 * bound + 1e-6)).max())
    print(f"[parity] {name}: max |err| {err.max():.3e}, worst err / allowed {ratio:.3f}", flush=True)
    return ratio
