"""Selected attention: each query token attends to the key blocks it selected (CPU, float64).
Test infrastructure only.

Sources: "FSA: An Alternative Efficient Implementation of Native Sparse Attention Kernel"
(Abstract) and the Flash-Sparse-Attention README page (overview, main features, the module's
configuration: block_size, topk, init_blocks, local_blocks, varlen cu_seqlens).  Native sparse
attention's selection branch: every query token selects top-k key blocks of block_size keys,
one selection per kv head shared by that head's group of query heads, and attends to the
union of the selected blocks.  FSA changes the loop order (key blocks outer, the queries that
selected a block gathered, then a reduction and an online-softmax pass), not the result, so
the result defined here is softmax attention over the selected key set.

Readings: selections are indices of key blocks within the token's own sequence; -1 marks an
unused slot; a token's selections are distinct (a repeated block is rejected).  Keys are
clipped to the sequence and, when causal, to keys <= position + (kv_len - q_len).  A token
with no visible key gets O = 0 and LSE = -inf, as everywhere in this library.
"""
from __future__ import annotations

import numpy as np

from .core import _attend, _kv_head, as_f64, default_scale


def _key_mask(sel_rows, q_len: int, kv_len: int, block_size: int, causal: bool) -> np.ndarray:
    """[q_len, kv_len] key sets of one (sequence, kv head) from sel_rows [q_len, topk]."""
    mask = np.zeros((q_len, kv_len), bool)
    for t in range(q_len):
        ents = [int(j) for j in sel_rows[t] if int(j) >= 0]
        if len(set(ents)) != len(ents):
            raise ValueError(f"token {t} selects a block twice: {ents}")
        for j in ents:
            if j * block_size >= kv_len:
                raise ValueError(f"block {j} lies past the sequence end")
            mask[t, j * block_size:min(kv_len, (j + 1) * block_size)] = True
    if causal:
        d = kv_len - q_len
        mask &= np.arange(kv_len)[None, :] <= np.arange(q_len)[:, None] + d
    return mask


def selected(q, k, v, sel, block_size: int, cu_seqlens_q=None, cu_seqlens_k=None, causal: bool = True,
             scale: float | None = None):
    """Fixed length: q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], sel [B,Sq,Hkv,topk] -> O [B,Sq,Hq,D],
    LSE [B,Hq,Sq].  Varlen (cu_seqlens given): q [Tq,Hq,D], k/v [Tk,Hkv,D], sel [Tq,Hkv,topk]
    -> O [Tq,Hq,D], LSE [Hq,Tq]."""
    q, k, v, sel = as_f64(q), as_f64(k), as_f64(v), np.asarray(sel)
    if cu_seqlens_q is None:
        B, Sq, Hq, D = q.shape
        cq = np.arange(B + 1) * Sq
        ck = np.arange(B + 1) * k.shape[1]
        o, lse = selected(q.reshape(B * Sq, Hq, D), k.reshape(-1, k.shape[2], D), v.reshape(-1, k.shape[2], D),
                          sel.reshape(B * Sq, sel.shape[2], sel.shape[3]), block_size, cq, ck, causal, scale)
        return o.reshape(B, Sq, Hq, D), lse.reshape(Hq, B, Sq).transpose(1, 0, 2)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = default_scale(D) if scale is None else scale
    o = np.zeros((Tq, Hq, D))
    lse = np.full((Hq, Tq), -np.inf)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        for hk in range(Hkv):
            mask = _key_mask(sel[q0:q1, hk], q1 - q0, k1 - k0, block_size, causal)
            for h in range(Hq):
                if _kv_head(h, Hq, Hkv) != hk:
                    continue
                o[q0:q1, h], lse[h, q0:q1] = _attend(q[q0:q1, h], k[k0:k1, hk], v[k0:k1, hk], mask, scale)
    return o, lse


def selected_rows(q, k, v, sel, block_size: int, cu_seqlens_q, cu_seqlens_k, b: int, h: int, rows,
                  causal: bool = True, scale: float | None = None):
    """Varlen spot check: (O [R, D], LSE [R]) for rows (positions within sequence b) of query
    head h, from that sequence's own keys only."""
    q, sel = np.asarray(q), np.asarray(sel)
    Tq, Hq, D = q.shape
    Hkv = np.asarray(k).shape[1]
    scale = default_scale(D) if scale is None else scale
    hk = _kv_head(h, Hq, Hkv)
    q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
    k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
    rows = np.asarray(rows)
    q_len, kv_len = q1 - q0, k1 - k0
    out_o = np.zeros((rows.size, D))
    out_l = np.zeros(rows.size)
    for n, r in enumerate(rows):
        m = _key_mask(sel[q0 + r:q0 + r + 1, hk], 1, kv_len, block_size, False)[0]
        if causal:
            m &= np.arange(kv_len) <= r + kv_len - q_len
        keys = np.nonzero(m)[0]
        oo, ll = _attend(as_f64(q[q0 + r:q0 + r + 1, h]), as_f64(np.asarray(k)[k0 + keys, hk]),
                         as_f64(np.asarray(v)[k0 + keys, hk]), np.ones((1, keys.size), bool), scale)
        out_o[n], out_l[n] = oo[0], ll[0]
    return out_o, out_l
