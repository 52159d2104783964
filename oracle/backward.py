"""Gradients of block-sparse attention (CPU, float64).  Test infrastructure only.

Source: the pages name a backward pass (the "Sparse FlashAttention with Incremental
Repair" README keeps FA's forward/backward kernels; the Flash-Sparse-Attention README and
FlagAttention's table list forward + backward for their sparse kernels) but print no
formula; the gradient of attention restricted to a key set is the plain derivative of the
forward in ``core``: with S = scale * Q K^T masked to the key set, P = softmax(S) row-wise,
O = P V and an upstream gradient dO,
  dV = P^T dO,   dP = dO V^T,   D_r = sum_d dO[r, d] O[r, d],
  dS = P * (dP - D)  (row-wise),   dQ = scale * dS K,   dK = scale * dS^T Q.
A row with no key has P = 0 and contributes nothing.  With grouped-query heads, a kv
head's dK and dV sum the contributions of its query heads.  With a softcap c the scores are
c tanh(S / c) (the forward's soft-capping), so dS is further multiplied by the derivative
1 - tanh(S / c)^2.
"""
from __future__ import annotations

import numpy as np

from .core import _kv_head, _list_head, as_f64, block_mask, causal_mask, default_scale


def _grads_head(q, k, v, do, mask, scale, softcap=0.0):
    x = scale * (q @ k.T)
    if softcap > 0.0:  # capped score c tanh(x / c); its derivative is 1 - tanh(x / c)^2
        t = np.tanh(x / softcap)
        x = softcap * t
    s = np.where(mask, x, -np.inf)
    m = s.max(axis=1, keepdims=True) if s.shape[1] else np.full((s.shape[0], 1), -np.inf)
    empty = np.isneginf(m)
    p = np.exp(s - np.where(empty, 0.0, m))
    l = p.sum(axis=1, keepdims=True)
    p = np.where(empty, 0.0, p / np.where(empty, 1.0, l))
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    dsum = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - dsum)
    if softcap > 0.0:
        ds = ds * (1.0 - t * t)
    return scale * (ds @ k), scale * (ds.T @ q), dv


def block_sparse_bwd(q, k, v, dout, count=None, index=None, block_M: int = 128, block_N: int = 128,
                     causal: bool = False, scale: float | None = None, softcap: float = 0.0):
    """dQ [B,Sq,Hq,D], dK and dV [B,Sk,Hkv,D] (float64) for the forward of ``core.block_sparse``
    (or dense attention when count is None), with the same softcap (0 = off)."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    scale = default_scale(D) if scale is None else scale
    cm = causal_mask(Sq, Sk) if causal else np.ones((Sq, Sk), bool)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            mask = cm.copy()
            if count is not None:
                ht = _list_head(h, Hq, Hkv, count.shape[1])
                mask &= block_mask(count[b, ht], index[b, ht], block_M, block_N, Sq, Sk)
            gq, gk, gv = _grads_head(q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h], mask, scale, softcap)
            dq[b, :, h] = gq
            dk[b, :, hk] += gk
            dv[b, :, hk] += gv
    return dq, dk, dv
