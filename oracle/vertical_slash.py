"""Vertical-slash index conversion and attention over it (CPU).  Test infrastructure only.

Source: "Implementation: Sgl project Sglang Sparse Flash Attention"
(Description, Signature, I/O Contract).  A vertical index is a key column
every query may attend to; a slash index is a diagonal.  The converter turns
per-(batch, head) raw indices into per-query-block metadata: block_count and
block_offset (ranges of keys that cover the slash diagonals) and column_count
and column_index (vertical columns), shaped (batch, heads, cdiv(context,
block_M)) and (..., NNZ_S) / (..., NNZ_V).  The page defers the algorithm to
another paper that is not among the sources, so the conversion below is this
library's own specification; its exact output (which covering windows are
chosen) is parity unpinned against the pages and pinned only by the coverage,
order and capacity invariants in the tests.

Conversion, for query block m of a sequence with q_len queries and kv_len
keys (d = kv_len - q_len, causal, rows r0 = m*block_M .. r1-1 with
r1 = min(r0 + block_M, q_len)); a slash offset s means key = row + d - s:

1. Walk the slash offsets in descending order, so the key ranges they cover
   in this block, [max(0, r0 + d - s), r1 - 1 + d - s], move rightwards.
   Ranges that end before key 0 are dropped.
2. Keep a frontier f (start: -infinity).  For a range [a, e]: if a >= f, open a
   window at a and set f = a + block_N; else if e >= f, open a window at f and
   set f = f + block_N; otherwise the range is already covered.
3. block_offset lists the window starts (key positions, ascending, disjoint
   windows of block_N keys); block_count is their number.
4. column_index lists, ascending, the vertical indices v <= r1 - 1 + d that no
   window contains; column_count is their number.
5. Query blocks past the end of the sequence (up to cdiv(context_size,
   block_M)) get counts 0.  Entries past a count are unspecified.

Attention over the metadata: row r of query block m attends to
(union of windows [w, w + block_N)  U  columns) intersected with [0, kv_len)
and, when causal, with keys <= r + d; then softmax attention as in ``core``.
"""
from __future__ import annotations

import numpy as np

from .core import _attend, as_f64, default_scale


def vs_convert_item(q_len: int, kv_len: int, vertical, slash, m: int, block_M: int, block_N: int):
    """Conversion for one (batch, head, query block).  Returns (windows, columns) as lists."""
    if block_M > block_N:
        raise ValueError("the conversion needs block_M <= block_N")
    r0 = m * block_M
    if r0 >= q_len:
        return [], []
    r1 = min(r0 + block_M, q_len)
    d = kv_len - q_len
    windows: list[int] = []
    frontier = None
    for s in sorted((int(x) for x in slash), reverse=True):
        e = r1 - 1 + d - s
        if e < 0:
            continue
        a = max(0, r0 + d - s)
        if frontier is None or a >= frontier:
            windows.append(a)
            frontier = a + block_N
        elif e >= frontier:
            windows.append(frontier)
            frontier += block_N
    last_visible = r1 - 1 + d
    covered = set()
    for w in windows:
        covered.update(range(w, w + block_N))
    columns = []
    for v in sorted(int(x) for x in vertical):
        if v > last_visible:
            break
        if v in covered:
            continue
        columns.append(v)
    return windows, columns


def vs_convert(q_seqlens, kv_seqlens, vertical, slash, context_size: int, block_M: int, block_N: int):
    """Full conversion for small inputs.

    vertical [B,H,NNZ_V], slash [B,H,NNZ_S] -> block_count [B,H,R], block_offset [B,H,R,NNZ_S],
    column_count [B,H,R], column_index [B,H,R,NNZ_V] with R = cdiv(context_size, block_M).
    Unused entries are -1.
    """
    vertical = np.asarray(vertical)
    slash = np.asarray(slash)
    B, H, nnz_v = vertical.shape
    nnz_s = slash.shape[2]
    R = (context_size + block_M - 1) // block_M
    bc = np.zeros((B, H, R), np.int32)
    bo = np.full((B, H, R, nnz_s), -1, np.int32)
    cc = np.zeros((B, H, R), np.int32)
    ci = np.full((B, H, R, nnz_v), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for m in range(R):
                w, c = vs_convert_item(int(q_seqlens[b]), int(kv_seqlens[b]), vertical[b, h], slash[b, h], m,
                                       block_M, block_N)
                bc[b, h, m] = len(w)
                bo[b, h, m, :len(w)] = w
                cc[b, h, m] = len(c)
                ci[b, h, m, :len(c)] = c
    return bc, bo, cc, ci


def vs_convert_mergehead(q_seqlens, kv_seqlens, vertical, slash, vertical_count, slash_count, context_size: int,
                         block_M: int, block_N: int):
    """Merged-head conversion ("Implementation: Sgl project Sglang Sparse Flash Attention",
    Description): per-head counts of valid indices.  Reading: vertical_count and slash_count
    have shape (H,), are shared by every batch entry, and head h uses the first count entries of
    its index rows (counts clamped to [0, NNZ]); the rest of the conversion is ``vs_convert``.
    Output shapes are those of ``vs_convert``."""
    vertical = np.asarray(vertical)
    slash = np.asarray(slash)
    B, H, nnz_v = vertical.shape
    nnz_s = slash.shape[2]
    R = (context_size + block_M - 1) // block_M
    bc = np.zeros((B, H, R), np.int32)
    bo = np.full((B, H, R, nnz_s), -1, np.int32)
    cc = np.zeros((B, H, R), np.int32)
    ci = np.full((B, H, R, nnz_v), -1, np.int32)
    for h in range(H):
        nv = min(max(int(vertical_count[h]), 0), nnz_v)
        ns = min(max(int(slash_count[h]), 0), nnz_s)
        for b in range(B):
            for m in range(R):
                w, c = vs_convert_item(int(q_seqlens[b]), int(kv_seqlens[b]), vertical[b, h, :nv],
                                       slash[b, h, :ns], m, block_M, block_N)
                bc[b, h, m] = len(w)
                bo[b, h, m, :len(w)] = w
                cc[b, h, m] = len(c)
                ci[b, h, m, :len(c)] = c
    return bc, bo, cc, ci


def _key_set(kv_len: int, windows, columns, block_N: int) -> np.ndarray:
    keys = set()
    for w in windows:
        keys.update(range(max(0, w), min(kv_len, w + block_N)))
    keys.update(c for c in columns if 0 <= c < kv_len)
    return np.array(sorted(keys), dtype=np.int64)


def vs_attention(q, k, v, block_count, block_offset, column_count, column_index, cu_seqlens_q, cu_seqlens_k,
                 block_M: int, block_N: int, causal: bool = True, scale: float | None = None,
                 softcap: float = 0.0):
    """Varlen attention over converted metadata (small inputs).

    q [total_q, H, D], k/v [total_k, Hk, D].  Returns O [total_q, H, D] and LSE [H, total_q].
    """
    q64, k64, v64 = as_f64(q), as_f64(k), as_f64(v)
    total_q, H, D = q64.shape
    Hk = k64.shape[1]
    scale = default_scale(D) if scale is None else scale
    o = np.zeros((total_q, H, D))
    lse = np.zeros((H, total_q))
    B = len(cu_seqlens_q) - 1
    for b in range(B):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        q_len, kv_len = q1 - q0, k1 - k0
        d = kv_len - q_len
        for h in range(H):
            hk = h // (H // Hk)
            for m in range((q_len + block_M - 1) // block_M):
                nb, nc = int(block_count[b, h, m]), int(column_count[b, h, m])
                keys = _key_set(kv_len, block_offset[b, h, m, :nb], column_index[b, h, m, :nc], block_N)
                rows = np.arange(m * block_M, min(q_len, (m + 1) * block_M))
                mask = np.ones((rows.size, keys.size), bool)
                if causal:
                    mask &= keys[None, :] <= rows[:, None] + d
                oo, ll = _attend(q64[q0 + rows, h], k64[k0 + keys, hk], v64[k0 + keys, hk], mask, scale,
                                 softcap)
                o[q0 + rows, h] = oo
                lse[h, q0 + rows] = ll
    return o, lse


def vs_attention_rows(q, k, v, b: int, h: int, rows, windows, columns, cu_seqlens_q, cu_seqlens_k,
                      block_N: int, causal: bool = True, scale: float | None = None, softcap: float = 0.0):
    """Attention for selected rows (local positions within sequence b) of one query block
    whose metadata (windows, columns) is given.  For full-size spot checks."""
    q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
    k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
    q_len, kv_len = q1 - q0, k1 - k0
    d = kv_len - q_len
    H, D = np.asarray(q).shape[1], np.asarray(q).shape[2]
    Hk = np.asarray(k).shape[1]
    scale = default_scale(D) if scale is None else scale
    hk = h // (H // Hk)
    keys = _key_set(kv_len, windows, columns, block_N)
    rows = np.asarray(rows)
    mask = np.ones((rows.size, keys.size), bool)
    if causal:
        mask &= keys[None, :] <= rows[:, None] + d
    return _attend(as_f64(np.asarray(q)[q0 + rows, h]), as_f64(np.asarray(k)[k0 + keys, hk]),
                   as_f64(np.asarray(v)[k0 + keys, hk]), mask, scale, softcap)
