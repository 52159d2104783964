"""The five synthetic workloads (and their scaled-down variants).

Each builder returns a plain dict of numpy arrays: bf16 tensors as uint16 bit
patterns in the layouts the library takes (q ``[B, Sq, Hq, D]``, k/v
``[B, Sk, Hkv, D]``, varlen ``[total, H, D]``), int32 index lists, and the
scalar parameters.  Nothing here computes attention; thresholds for the gated
workload are picked from tile maxima that the caller supplies.

Seeds: workload n (1-based) uses seed ``1000 + n`` unless a test passes its own.
"""
from __future__ import annotations

import numpy as np

from . import f32_to_bf16_bits, normal_bf16, normal_f32, power_law_unique, random_subset_sorted, rng


# ---------------------------------------------------------------------------
# Query construction shared by the prefill workloads
# ---------------------------------------------------------------------------

def spiked_queries(seed: int, tag: str, B: int, S: int, H: int, D: int,
                   rank: int = 4, prob: float = 0.125, amp: float = 16.0) -> np.ndarray:
    """Q ~ N(0, 1) plus planted low-rank spikes, rounded to bf16.

    Per head, ``rank`` random unit directions are drawn; each row gets
    ``amp * u_r`` added (r uniform) with probability ``prob``.
    """
    q = normal_f32(seed, tag + ".base", (B, S, H, D))
    g = rng(seed, tag + ".spikes")
    u = g.standard_normal((H, rank, D)).astype(np.float64)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    hit = g.random((B, S, H)) < prob
    which = g.integers(0, rank, size=(B, S, H))
    hidx = np.broadcast_to(np.arange(H)[None, None, :], (B, S, H))
    add = (amp * u[hidx, which]).astype(np.float32)          # [B, S, H, D]
    q = q + np.where(hit[..., None], add, np.float32(0.0))
    return f32_to_bf16_bits(q)


# ---------------------------------------------------------------------------
# Workload 1: tiny sparse decode
# ---------------------------------------------------------------------------

def tiny_decode(seed: int = 1001, B: int = 1, H: int = 4, D: int = 64, Sk: int = 1024,
                bs: int = 64, n_a: int = 6) -> dict:
    """Sq = 1, Hq = Hkv = H.  Per (b, h): set A = n_a random blocks, set B = the rest."""
    nkb = Sk // bs
    q = normal_bf16(seed, "q", (B, 1, H, D))
    k = normal_bf16(seed, "k", (B, Sk, H, D))
    v = normal_bf16(seed, "v", (B, Sk, H, D))
    g = rng(seed, "lists")
    set_a = np.zeros((B, H, n_a), np.int32)
    set_b = np.zeros((B, H, nkb - n_a), np.int32)
    for b in range(B):
        for h in range(H):
            a = random_subset_sorted(g, nkb, n_a)
            set_a[b, h] = a
            set_b[b, h] = np.setdiff1d(np.arange(nkb, dtype=np.int32), a)
    full = np.broadcast_to(np.arange(nkb, dtype=np.int32), (B, H, nkb)).copy()
    return dict(q=q, k=k, v=v, set_a=set_a, set_b=set_b, full=full, B=B, Hq=H, Hkv=H,
                Sq=1, Sk=Sk, D=D, block_size=bs)


# ---------------------------------------------------------------------------
# Workload 2: speculative + sparse decode
# ---------------------------------------------------------------------------

def spec_sparse_decode(seed: int = 1002, B: int = 32, Hq: int = 32, Hkv: int = 8, D: int = 128,
                       Sk: int = 32768, bs: int = 64, spec_tokens: int = 2048,
                       frac: float = 0.25) -> dict:
    """Pass 1 = the last ``spec_tokens`` keys (dense, causal); pass 2 = ``frac`` of the
    earlier ``bs``-token blocks, chosen at random per (b, h_kv), ascending."""
    nkb = Sk // bs
    n_spec_blocks = spec_tokens // bs
    n_early = nkb - n_spec_blocks
    n_missed = int(round(frac * n_early))
    q = normal_bf16(seed, "q", (B, 1, Hq, D))
    k = normal_bf16(seed, "k", (B, Sk, Hkv, D))
    v = normal_bf16(seed, "v", (B, Sk, Hkv, D))
    g = rng(seed, "missed")
    missed = np.zeros((B, Hkv, n_missed), np.int32)
    for b in range(B):
        for h in range(Hkv):
            missed[b, h] = random_subset_sorted(g, n_early, n_missed)
    return dict(q=q, k=k, v=v, missed=missed, spec_start=n_early * bs, B=B, Hq=Hq, Hkv=Hkv,
                Sq=1, Sk=Sk, D=D, block_size=bs)


# ---------------------------------------------------------------------------
# Workload 3: block-sparse causal prefill
# ---------------------------------------------------------------------------

def block_sparse_prefill(seed: int = 1003, B: int = 1, Hq: int = 32, Hkv: int = 8, S: int = 32768,
                         D: int = 128, bs: int = 128, n_random: int = 32) -> dict:
    """Per (b, h_q, query block i): {i} U {0} U n_random distinct blocks from 1..i-1."""
    nqb = S // bs
    q = spiked_queries(seed, "q", B, S, Hq, D)
    k = normal_bf16(seed, "k", (B, S, Hkv, D))
    v = normal_bf16(seed, "v", (B, S, Hkv, D))
    cap = n_random + 2
    count = np.zeros((B, Hq, nqb), np.int32)
    index = np.zeros((B, Hq, nqb, cap), np.int32)
    g = rng(seed, "lists")
    for b in range(B):
        for h in range(Hq):
            for i in range(nqb):
                if i == 0:
                    sel = np.array([0], np.int32)
                elif i - 1 <= n_random:
                    sel = np.arange(i + 1, dtype=np.int32)
                else:
                    mid = g.choice(np.arange(1, i), size=n_random, replace=False)
                    sel = np.sort(np.concatenate([[0], mid, [i]])).astype(np.int32)
                count[b, h, i] = sel.size
                index[b, h, i, :sel.size] = sel
    return dict(q=q, k=k, v=v, count=count, index=index, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Sk=S, D=D,
                block_M=bs, block_N=bs, cap=cap)


# ---------------------------------------------------------------------------
# Workload 4: BSFA gated prefill
# ---------------------------------------------------------------------------

def gated_prefill(seed: int = 1004, B: int = 1, Hq: int = 32, Hkv: int = 8, S: int = 65536,
                  D: int = 128, bs: int = 128, kscale_sigma: float = 0.25) -> dict:
    """Q as the block-sparse workload; V ~ N(0,1); K ~ N(0,1) times a per-(h_kv, key block)
    factor exp(sigma * z), which spreads the tile maxima.  Thresholds are chosen later
    from tile maxima (``thresholds_from_tile_max``)."""
    nkb = S // bs
    q = spiked_queries(seed, "q", B, S, Hq, D)
    kn = normal_f32(seed, "k", (B, S, Hkv, D))
    z = rng(seed, "kscale").standard_normal((B, nkb, Hkv)).astype(np.float32)
    fac = np.exp(np.float32(kscale_sigma) * z)                          # [B, nkb, Hkv]
    kn = kn.reshape(B, nkb, bs, Hkv, D) * fac[:, :, None, :, None]
    k = f32_to_bf16_bits(kn.reshape(B, S, Hkv, D))
    v = normal_bf16(seed, "v", (B, S, Hkv, D))
    return dict(q=q, k=k, v=v, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Sk=S, D=D, block_M=bs, block_N=bs)


def thresholds_from_tile_max(tmax_row: np.ndarray, i: int, min_gap: float = 2e-2,
                             target: float = 0.5) -> float:
    """Pick T for query block i from the tile maxima of its off-diagonal tiles.

    ``tmax_row[j]`` for j < i are the (scaled) tile maxima.  Candidate
    thresholds are the midpoints of gaps of at least ``min_gap`` between
    consecutive sorted maxima (plus one below the minimum and one above the
    maximum); the one whose split rank is nearest ``target`` skipped is taken.
    Every returned T is at least min_gap/2 away from each maximum.  i = 0 has
    no off-diagonal tiles and gets -inf.
    """
    if i == 0:
        return float("-inf")
    t = np.sort(np.asarray(tmax_row[:i], dtype=np.float64))
    cands = [(0, t[0] - min_gap)]                      # rank = number of tiles below T
    for r in range(1, t.size):
        if t[r] - t[r - 1] >= min_gap:
            cands.append((r, 0.5 * (t[r] + t[r - 1])))
    cands.append((t.size, t[-1] + min_gap))
    best = min(cands, key=lambda c: (abs(c[0] / t.size - target), c[0]))
    return float(np.float32(best[1]))


# ---------------------------------------------------------------------------
# Workload 5: vertical-slash varlen prefill
# ---------------------------------------------------------------------------

def vs_varlen_prefill(seed: int = 1005, seqlens=(65536, 32768), H: int = 32, D: int = 128,
                      nnz_v: int = 1000, nnz_s: int = 2000, block: int = 64,
                      context_size: int | None = None, with_tensors: bool = True) -> dict:
    """Packed varlen Q/K/V ``[total, H, D]``; per (b, h) ``nnz_v`` vertical key indices
    (ascending) and ``nnz_s`` slash offsets (descending), power-law sampled with 0 forced.
    A slash offset s marks the diagonal key = query + (kv_len - q_len) - s.
    ``with_tensors=False`` leaves Q/K/V out (None); the indices are the same either way."""
    seqlens = [int(s) for s in seqlens]
    B = len(seqlens)
    total = int(sum(seqlens))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    q = k = v = None
    if with_tensors:
        q = normal_bf16(seed, "q", (total, H, D))
        k = normal_bf16(seed, "k", (total, H, D))
        v = normal_bf16(seed, "v", (total, H, D))
    vert = np.zeros((B, H, nnz_v), np.int32)
    slash = np.zeros((B, H, nnz_s), np.int32)
    for b in range(B):
        L = seqlens[b]
        for h in range(H):
            gv = rng(seed, f"vertical.{b}.{h}")
            gs = rng(seed, f"slash.{b}.{h}")
            # a sequence shorter than the index count is padded with positions >= L, which no
            # row of that sequence can reach (keeps the lists unique and sorted)
            vv = np.sort(power_law_unique(gv, L, nnz_v))
            vert[b, h] = np.concatenate([vv, L + np.arange(nnz_v - vv.size)])
            ss = np.sort(power_law_unique(gs, L, nnz_s))[::-1]
            slash[b, h] = np.concatenate([L + np.arange(nnz_s - ss.size)[::-1], ss])
    if context_size is None:
        context_size = max(seqlens)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, seqlens=np.array(seqlens, np.int32), vertical=vert,
                slash=slash, B=B, H=H, D=D, block_M=block, block_N=block,
                context_size=int(context_size), max_seqlen=max(seqlens))


# ---------------------------------------------------------------------------
# Selected attention (top-k key blocks per query token), the FSA module's example shape
# ---------------------------------------------------------------------------

def selected_prefill(seed: int = 1006, seqlens=(65536, 32768), Hq: int = 4, Hkv: int = 4, D: int = 128,
                     block: int = 64, topk: int = 16, init_blocks: int = 1, local_blocks: int = 2) -> dict:
    """Packed varlen Q/K/V ``[total, H, D]`` ~ N(0, 1) and per (token, kv head) a selection of
    up to ``topk`` distinct key blocks of its own sequence, ``sel [total, Hkv, topk]`` int32:
    the first ``init_blocks`` blocks, the ``local_blocks`` blocks ending at the token's own
    block, and uniformly random other causally reachable blocks to fill ``topk``; -1 pads a
    token that can reach fewer blocks.  Slot order is random."""
    seqlens = [int(s) for s in seqlens]
    total = int(sum(seqlens))
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    q = normal_bf16(seed, "q", (total, Hq, D))
    k = normal_bf16(seed, "k", (total, Hkv, D))
    v = normal_bf16(seed, "v", (total, Hkv, D))
    sel = np.full((total, Hkv, topk), -1, np.int32)
    g = rng(seed, "sel")
    chunk = 8192
    for b, L in enumerate(seqlens):
        for p0 in range(0, L, chunk):
            pos = np.arange(p0, min(L, p0 + chunk))
            own = pos // block                                   # the token's own block
            nb = own + 1                                         # causally reachable blocks
            R = pos.size
            for hk in range(Hkv):
                fixed = np.full((R, init_blocks + local_blocks), -1, np.int64)
                fixed[:, :init_blocks] = np.arange(init_blocks)[None, :]
                fixed[:, init_blocks:] = own[:, None] - np.arange(local_blocks)[None, ::-1]
                fixed = np.where((fixed >= 0) & (fixed < nb[:, None]), fixed, -1)
                # dedupe: a local block that is also an init block counts once
                for c in range(init_blocks, init_blocks + local_blocks):
                    fixed[:, c] = np.where(fixed[:, c] < init_blocks, -1, fixed[:, c])
                # random others from [init_blocks, own - local_blocks + 1)
                lo = init_blocks
                hi = np.maximum(own - local_blocks + 1, lo)               # exclusive
                n_rand = topk - (fixed >= 0).sum(axis=1)
                span = hi - lo
                width = int(span.max()) if R else 0
                picks = np.full((R, topk), -1, np.int64)
                if width > 0:
                    keys = g.random((R, width))
                    keys[np.arange(width)[None, :] >= span[:, None]] = np.inf
                    m = min(topk, width)
                    order = np.argsort(keys, axis=1)[:, :m]
                    take = np.arange(m)[None, :] < np.minimum(n_rand, span)[:, None]
                    picks[:, :m] = np.where(take, order + lo, -1)
                allsel = np.concatenate([fixed, picks], axis=1)
                # compact the valid entries to the front, then shuffle the slots
                valid = allsel >= 0
                idx = np.argsort(~valid, axis=1, kind="stable")[:, :topk]
                row = np.take_along_axis(allsel, idx, axis=1)
                perm = np.argsort(g.random((R, topk)), axis=1)
                sel[cu[b] + pos, hk] = np.take_along_axis(row, perm, axis=1)
    return dict(q=q, k=k, v=v, sel=sel, cu_seqlens=cu, seqlens=np.array(seqlens, np.int32), Hq=Hq, Hkv=Hkv,
                D=D, block=block, topk=topk, max_seqlen=max(seqlens))
