"""BSFA tile-maximum gating (float64, CPU).  Test infrastructure only.

Definition followed: "Block Sparse Flash Attention", Abstract and Figure 2
(mechanism).  Inside the FlashAttention tile loop the exact per-tile maximum
score s_max^(i,j) of query block i against key block j is compared with a
calibrated threshold T(h, i) (one value per query block of a head; -inf keeps
every tile).  Off-diagonal tiles are kept when s_max >= T; the diagonal tile
always runs; a skipped tile contributes neither the V_j load nor the P V_j
product.

Readings (the page leaves these open):
* Causal self-attention only (Sq == Sk), square tiles; tiles j > i are never
  visited.
* What a skipped tile leaves in the softmax.  Figure 2 lists what a skipped
  block avoids, the V_j load and the P V_j product, and says nothing of the
  running maximum and normaliser, which the tile's scores (computed anyway for
  s_max) could still feed.  Both readings are implemented (``skipped``):
  - "drop" (default): the scores are left out altogether, so the gated result
    is exactly block-sparse attention over the kept tiles (the top-k "value
    blocks" of the Abstract are then the only blocks attended);
  - "count": the literal reading of Figure 2, in which only the V_j load and the
    product are skipped.  The tile's scores stay in the maximum and in the
    normaliser, which is then attention over every causal key with the value
    rows of skipped tiles taken as zero.  LSE is then the dense causal LSE
    whatever the thresholds.
  Which one the page's kernel runs is parity unpinned against the pages.  Each
  is pinned through its own closed forms: "drop" equals block-sparse attention
  over the kept tiles; "count" has the dense causal LSE, and its numerator
  O*exp(LSE) equals that of "drop".
* The scores are the scaled dot products scale*<q, k>; the comparison is taken
  in float32, the precision of the kernel: the exact float64 tile maximum is
  rounded to float32 and compared with the float32 threshold.

Threshold calibration (same page, Abstract: a one-time calibration on a small
data set learns per-layer and per-head score distributions so that the top-k
blocks of each query are kept; Figure 2: one threshold T^(k) per query row,
-inf where fewer than k off-diagonal candidates exist).  The page gives no
procedure; reading taken here: for each calibration sample b, head h and query
block i, the k-th largest off-diagonal tile maximum t(i, j), j < i; -inf when
i < k; T(h, i) is the mean of those values over the samples.  Gating one
sample with its own threshold then keeps exactly min(k, i) off-diagonal tiles
of each row (ties aside); the target density of row i is (min(k, i) + 1) /
(i + 1), the diagonal included.
"""
from __future__ import annotations

import numpy as np

from .core import _attend, _kv_head, as_f64, default_scale


def _check(Sq: int, Sk: int, BM: int, BN: int) -> None:
    if Sq != Sk or BM != BN or Sq % BM:
        raise ValueError("gating needs Sq == Sk, square tiles and Sq divisible by the tile")


def tile_max_row(q, k, b: int, h: int, i: int, BM: int, BN: int, scale: float | None = None):
    """Scaled tile maxima t(i, j) for j = 0..i of head h (float64).

    t(i, i) is taken over the causally visible entries of the diagonal tile.
    """
    q, k = np.asarray(q), np.asarray(k)
    Hq, D = q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    scale = default_scale(D) if scale is None else scale
    hk = _kv_head(h, Hq, Hkv)
    qi = as_f64(q[b, i * BM:(i + 1) * BM, h])                 # [BM, D]
    kk = as_f64(k[b, :(i + 1) * BN, hk])                       # [(i+1)BN, D]
    s = scale * (qi @ kk.T)                                    # [BM, (i+1)BN]
    r = np.arange(BM)[:, None] + i * BM
    c = np.arange((i + 1) * BN)[None, :]
    s = np.where(c <= r, s, -np.inf)
    return s.reshape(BM, i + 1, BN).max(axis=(0, 2))


def _keep_row(t: np.ndarray, T: float, i: int) -> np.ndarray:
    """Keep decisions for query block i: float32(t) >= float32(T); diagonal always kept."""
    keep = (t.astype(np.float32) >= np.float32(T)).astype(np.uint8)
    keep[i] = 1
    return keep


def _skip_check(skipped: str) -> None:
    if skipped not in ("drop", "count"):
        raise ValueError('skipped must be "drop" or "count"')


def gated(q, k, v, T, BM: int = 128, BN: int = 128, scale: float | None = None, skipped: str = "drop"):
    """Gated causal attention for small inputs.

    q [B,S,Hq,D], k/v [B,S,Hkv,D], T [B,Hq,nQB] (float32 thresholds).
    skipped: "drop" (a skipped tile is left out of the softmax) or "count" (its scores stay
    in the maximum and the normaliser, its values do not enter O).
    Returns O [B,S,Hq,D], LSE [B,Hq,S], keep [B,Hq,nQB,nKB] (uint8, 0 above the
    diagonal) and tmax [B,Hq,nQB,nKB] (float64, NaN above the diagonal).
    """
    _skip_check(skipped)
    B, S, Hq, D = np.asarray(q).shape
    Hkv = np.asarray(k).shape[2]
    _check(S, np.asarray(k).shape[1], BM, BN)
    scale = default_scale(D) if scale is None else scale
    nqb = S // BM
    o = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, Hq, S))
    keep = np.zeros((B, Hq, nqb, nqb), np.uint8)
    tmax = np.full((B, Hq, nqb, nqb), np.nan)
    vv = as_f64(v)
    qq = as_f64(q)
    kk = as_f64(k)
    for b in range(B):
        for h in range(Hq):
            hk = _kv_head(h, Hq, Hkv)
            mask = np.zeros((S, S), bool)
            for i in range(nqb):
                t = tile_max_row(q, k, b, h, i, BM, BN, scale)
                tmax[b, h, i, :i + 1] = t
                kr = _keep_row(t, T[b, h, i], i)
                keep[b, h, i, :i + 1] = kr
                if skipped == "count":
                    rows = np.arange(i * BM, (i + 1) * BM)
                    o[b, rows, h], lse[b, h, rows] = _attend_counting_skipped(
                        qq[b, rows, h], kk[b, :, hk], vv[b, :, hk], rows, kr, BN, scale)
                for j in np.nonzero(kr)[0]:
                    mask[i * BM:(i + 1) * BM, j * BN:(j + 1) * BN] = True
            if skipped == "drop":
                mask &= np.arange(S)[None, :] <= np.arange(S)[:, None]
                o[b, :, h], lse[b, h] = _attend(qq[b, :, h], kk[b, :, hk], vv[b, :, hk], mask, scale)
    return o, lse, keep, tmax


def _attend_counting_skipped(q_rows, k, v, rows, keep_row, BN: int, scale: float):
    """Rows of one query block (all of whose keys j <= i tiles are causal candidates) under the
    "count" reading: softmax over every causal key, values of skipped tiles taken as zero."""
    nk = keep_row.size * BN
    kept_key = np.repeat(keep_row.astype(bool), BN)             # [nk]
    v0 = np.where(kept_key[:, None], v[:nk], 0.0)
    mask = np.arange(nk)[None, :] <= np.asarray(rows)[:, None]
    return _attend(q_rows, k[:nk], v0, mask, scale)


def gated_rows(q, k, v, T: float, b: int, h: int, i: int, rows, BM: int = 128, BN: int = 128,
               scale: float | None = None, skipped: str = "drop"):
    """Gated attention for selected rows of query block i of head h (full-size spot checks).

    Returns (O [R, D], LSE [R], keep row [i+1], t row [i+1]).
    """
    _skip_check(skipped)
    q, k = np.asarray(q), np.asarray(k)
    Hq, D = q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    scale = default_scale(D) if scale is None else scale
    hk = _kv_head(h, Hq, Hkv)
    t = tile_max_row(q, k, b, h, i, BM, BN, scale)
    kr = _keep_row(t, T, i)
    if skipped == "count":
        nk = (i + 1) * BN
        o, lse = _attend_counting_skipped(as_f64(q[b, np.asarray(rows), h]), as_f64(k[b, :nk, hk]),
                                          as_f64(v[b, :nk, hk]), rows, kr, BN, scale)
        return o, lse, kr, t
    kept = np.nonzero(kr)[0]
    cols = np.concatenate([np.arange(j * BN, (j + 1) * BN) for j in kept])
    kv = as_f64(k[b, cols, hk])
    vv = as_f64(v[b, cols, hk])
    rows = np.asarray(rows)
    qr = as_f64(q[b, rows, h])
    mask = cols[None, :] <= rows[:, None]
    o, lse = _attend(qr, kv, vv, mask, scale)
    return o, lse, kr, t


def calibrate(q, k, k_keep: int, BM: int = 128, BN: int = 128, scale: float | None = None):
    """Thresholds T [Hq, nQB] (float64; -inf where i < k_keep) from the calibration samples
    q [B,S,Hq,D], k [B,S,Hkv,D], and the per-sample values [B, Hq, nQB]."""
    if k_keep < 1:
        raise ValueError("k_keep must be at least 1")
    B, S, Hq, _ = np.asarray(q).shape
    _check(S, np.asarray(k).shape[1], BM, BN)
    nqb = S // BM
    per = np.full((B, Hq, nqb), -np.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(k_keep, nqb):
                t = tile_max_row(q, k, b, h, i, BM, BN, scale)[:i]   # off-diagonal candidates
                per[b, h, i] = np.sort(t)[::-1][k_keep - 1]
    return per.mean(axis=0), per


def density(keep, k_keep: int):
    """(realised, target) fraction of causal tiles kept, over every (b, h, query block) row of a
    keep mask [B, Hq, nQB, nKB]; the target of row i is (min(k_keep, i) + 1) / (i + 1)."""
    keep = np.asarray(keep)
    nqb = keep.shape[-2]
    lower = np.tril(np.ones((nqb, nqb), bool))
    realised = float(keep[..., lower].sum()) / (keep[..., 0, 0].size * lower.sum())
    i = np.arange(nqb)
    target = float(np.sum(np.minimum(k_keep, i) + 1)) / lower.sum()
    return realised, target
