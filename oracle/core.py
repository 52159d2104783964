"""Block-sparse softmax attention, partials and the log-sum-exp combine (float64, CPU).

Test infrastructure only (see the package docstring).

Definitions followed:

* Attention restricted to a key set.  "Sparse FlashAttention with Incremental
  Repair" (README, Usage, section 1: sparse-only forward): each table entry
  names a block of ``block_size`` consecutive keys at offset
  ``index * block_size``; the output is softmax attention over exactly those
  keys, ``out`` shaped like q and ``lse`` of shape (B, H, Sq); an empty
  table gives out = 0 and lse = -inf.  For a row r with key set K(r):
  s_k = scale * <q_r, k_k>, m = max s, l = sum exp(s_k - m),
  O_r = sum exp(s_k - m) v_k / l, LSE_r = m + ln l (natural log).
* Default scale 1/sqrt(head_dim): "Sglang Sparse Flash Attention",
  I/O Contract (softmax_scale).
* Softcap: same page, Signature and I/O Contract (softcap, 0.0 switches it
  off).  The page gives no formula; reading: the usual logit soft-capping,
  applied to the scaled score before the softmax,
  s_k = softcap * tanh(scale * <q_r, k_k> / softcap).
* Grouped-query heads: q has H heads, k/v have Hk heads (same pages, shapes);
  query head h reads key/value head floor(h / (H / Hk)).
* Causal masking, where asked for, is bottom-right aligned: key c is visible
  to row r iff c <= r + (Sk - Sq).  (The pages give no alignment; with one
  decode query this reading lets it see the whole cache.)
* Combine: "Sparse FlashAttention with Incremental Repair", What's in this
  fork (validated combine identity FA(A u B) == Combine(FA(A), FA(B))) and
  Usage section 2.  For partials (o_p, lse_p): m = max lse_p; if m = -inf the
  result is (0, -inf); otherwise w_p = exp(lse_p - m),
  O = sum w_p o_p / sum w_p, LSE = m + ln sum w_p.
* Per-entry partials: same page, Usage section 3: one (o, lse) per table
  entry; entries past a list's count are the neutral partial (0, -inf).
* Speculative + sparse: same page, Usage section 2: attention over the
  speculative keys (optionally causal), attention over the missed blocks
  (never masked), then the combine.
"""
from __future__ import annotations

import math

import numpy as np


def as_f64(x) -> np.ndarray:
    """bf16 bit patterns (uint16) or any float array -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def causal_mask(Sq: int, Sk: int) -> np.ndarray:
    """[Sq, Sk] bool: key c visible to row r iff c <= r + (Sk - Sq)."""
    r = np.arange(Sq)[:, None]
    c = np.arange(Sk)[None, :]
    return c <= r + (Sk - Sq)


def block_mask(count: np.ndarray, index: np.ndarray, block_M: int, block_N: int, Sq: int,
               Sk: int) -> np.ndarray:
    """[Sq, Sk] bool key sets for one (batch, head) from per-query-block lists.

    ``count[i]`` entries of ``index[i]`` are the key blocks of query block i.
    Block j covers keys [j*block_N, (j+1)*block_N) clipped to [0, Sk).
    Duplicate entries are rejected (lists are sets).
    """
    mask = np.zeros((Sq, Sk), dtype=bool)
    nqb = (Sq + block_M - 1) // block_M
    for i in range(nqb):
        ents = [int(j) for j in index[i, :int(count[i])]]
        if len(set(ents)) != len(ents):
            raise ValueError(f"duplicate block in list of query block {i}: {ents}")
        r0, r1 = i * block_M, min(Sq, (i + 1) * block_M)
        for j in ents:
            if not 0 <= j * block_N < Sk:
                raise ValueError(f"block {j} out of range")
            mask[r0:r1, j * block_N:min(Sk, (j + 1) * block_N)] = True
    return mask


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float, softcap: float = 0.0):
    """Softmax attention of rows q [R, D] over keys k/v [Sk, D] restricted by mask [R, Sk]."""
    s = scale * (q @ k.T)
    if softcap > 0.0:
        s = softcap * np.tanh(s / softcap)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = np.isneginf(m)
    m0 = np.where(empty, 0.0, m)
    p = np.exp(s - m0[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / np.where(empty, 1.0, l)[:, None]
    o[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m0 + np.log(np.where(empty, 1.0, l)))
    return o, lse


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    return h // (Hq // Hkv)


def _list_head(h: int, Hq: int, Hkv: int, Ht: int) -> int:
    if Ht == Hq:
        return h
    if Ht == Hkv:
        return _kv_head(h, Hq, Hkv)
    raise ValueError("list heads must equal Hq or Hkv")


def dense(q, k, v, causal: bool = False, scale: float | None = None, softcap: float = 0.0):
    """Dense attention.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] -> (O [B,Sq,Hq,D], LSE [B,Hq,Sq])."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    scale = default_scale(D) if scale is None else scale
    mask = causal_mask(Sq, Sk) if causal else np.ones((Sq, Sk), bool)
    o = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            o[b, :, h], lse[b, h] = _attend(q[b, :, h], k[b, :, hk], v[b, :, hk], mask, scale, softcap)
    return o, lse


def block_sparse(q, k, v, count, index, block_M: int, block_N: int, causal: bool = False,
                 scale: float | None = None, softcap: float = 0.0):
    """Attention over per-(b, list head, query block) block lists.

    count [B, Ht, nQB], index [B, Ht, nQB, cap]; Ht is Hq (a list per query
    head) or Hkv (one list shared by a group of query heads).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    Ht = count.shape[1]
    scale = default_scale(D) if scale is None else scale
    cm = causal_mask(Sq, Sk) if causal else None
    o = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            ht = _list_head(h, Hq, Hkv, Ht)
            hk = _kv_head(h, Hq, Hkv)
            mask = block_mask(count[b, ht], index[b, ht], block_M, block_N, Sq, Sk)
            if cm is not None:
                mask &= cm
            o[b, :, h], lse[b, h] = _attend(q[b, :, h], k[b, :, hk], v[b, :, hk], mask, scale, softcap)
    return o, lse


def block_sparse_partials(q, k, v, count, index, block_M: int, block_N: int, causal: bool = False,
                          scale: float | None = None, softcap: float = 0.0):
    """One (o, lse) per list entry.  Returns o_part [cap,B,Sq,Hq,D], lse_part [cap,B,Hq,Sq];
    entry e of a list with fewer than e+1 entries is (0, -inf)."""
    cap = index.shape[-1]
    q64 = as_f64(q)
    B, Sq, Hq, D = q64.shape
    o_part = np.zeros((cap, B, Sq, Hq, D))
    lse_part = np.full((cap, B, Hq, Sq), -np.inf)
    for e in range(cap):
        cnt_e = (count > e).astype(np.int32)
        idx_e = np.zeros(index.shape[:-1] + (1,), np.int32)
        idx_e[..., 0] = np.where(count > e, index[..., e], 0)
        o_part[e], lse_part[e] = block_sparse(q, k, v, cnt_e, idx_e, block_M, block_N, causal, scale,
                                                  softcap)
    return o_part, lse_part


def combine(o_part, lse_part):
    """Log-sum-exp merge of partials o_part [P,B,Sq,H,D], lse_part [P,B,H,Sq]."""
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    lse_t = np.transpose(lse_part, (0, 1, 3, 2))              # [P, B, Sq, H]
    m = lse_t.max(axis=0)                                      # [B, Sq, H]
    empty = np.isneginf(m)
    m0 = np.where(empty, 0.0, m)
    w = np.exp(lse_t - m0[None])                               # 0 for -inf partials
    wsum = w.sum(axis=0)
    o = (w[..., None] * o_part).sum(axis=0) / np.where(empty, 1.0, wsum)[..., None]
    o[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m0 + np.log(np.where(empty, 1.0, wsum)))
    return o, np.transpose(lse, (0, 2, 1))


def speculative_sparse(q, k_spec, v_spec, k, v, missed_count, missed_index, block_size: int,
                       causal_spec: bool = True, scale: float | None = None, softcap: float = 0.0):
    """Dense attention over (k_spec, v_spec), sparse attention over the missed blocks of
    (k, v) without a mask, then the combine of the two partials."""
    o1, l1 = dense(q, k_spec, v_spec, causal=causal_spec, scale=scale, softcap=softcap)
    Sq = np.asarray(q).shape[1]
    o2, l2 = block_sparse(q, k, v, missed_count, missed_index, max(Sq, 1), block_size, False, scale, softcap)
    return combine(np.stack([o1, o2]), np.stack([l1, l2]))


def attend_rows(q_rows, k, v, key_sets, scale: float, softcap: float = 0.0):
    """Attention for individual rows: q_rows [R, D]; k/v [Sk, D] of the row's kv head;
    key_sets a list of R integer arrays.  For spot checks at full size."""
    q_rows, k, v = as_f64(q_rows), as_f64(k), as_f64(v)
    R = q_rows.shape[0]
    o = np.zeros((R, q_rows.shape[1]))
    lse = np.zeros(R)
    for r in range(R):
        ks = np.asarray(key_sets[r], dtype=np.int64)
        if len(np.unique(ks)) != len(ks):
            raise ValueError("duplicate keys in a key set")
        mask = np.ones((1, ks.size), bool)
        o[r], lse[r] = (x[0] for x in _attend(q_rows[r:r + 1], k[ks], v[ks], mask, scale, softcap))
    return o, lse
