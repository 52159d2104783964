"""Pins for the float64 oracle's core: attention over key sets, block lists, partials, combine.

Each test checks the oracle against something other than itself: an independent
library routine (torch scaled_dot_product_attention in float64, scipy logsumexp),
a closed form, an invariant the pages state, or pure-Python brute force.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from synth import bf16_to_f64, normal_bf16, rng

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in float64.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] as float64 numpy."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal,
                                                         enable_gqa=tq.shape[1] != tk.shape[1])
    return o.permute(0, 2, 1, 3).numpy()


def _lse_ref(q, k, mask, Hq, Hkv):
    """logsumexp of the scaled masked scores via scipy, [B, Hq, Sq]."""
    D = q.shape[-1]
    B, Sq = q.shape[0], q.shape[1]
    out = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            s = (q[b, :, h] @ k[b, :, h // (Hq // Hkv)].T) / math.sqrt(D)
            s = np.where(mask, s, -np.inf)
            out[b, h] = logsumexp(s, axis=1)
    return out


def _inputs(seed, B, Sq, Sk, Hq, Hkv, D):
    q = normal_bf16(seed, "q", (B, Sq, Hq, D))
    k = normal_bf16(seed, "k", (B, Sk, Hkv, D))
    v = normal_bf16(seed, "v", (B, Sk, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 4, False), (4, 2, True), (6, 2, False), (2, 1, True)])
def test_dense_matches_torch_sdpa(Hq, Hkv, causal):
    q, k, v = _inputs(1, 2, 40, 40, Hq, Hkv, 16)
    o, lse = oracle.dense(q, k, v, causal=causal)
    qf, kf, vf = bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v)
    ref = _sdpa(qf, kf, vf, causal=causal)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    mask = np.tril(np.ones((40, 40), bool)) if causal else np.ones((40, 40), bool)
    np.testing.assert_allclose(lse, _lse_ref(qf, kf, mask, Hq, Hkv), atol=1e-12, rtol=0)


def test_brute_force_tiny():
    """Pure-Python loops with math.exp / math.fsum on a tiny irregular key set."""
    q, k, v = _inputs(2, 1, 3, 11, 1, 1, 5)
    qf, kf, vf = bf16_to_f64(q)[0, :, 0], bf16_to_f64(k)[0, :, 0], bf16_to_f64(v)[0, :, 0]
    sets = [[0, 3, 7], [10], [1, 2, 4, 5, 6, 8, 9]]
    o, lse = oracle.attend_rows(qf, kf, vf, sets, 1 / math.sqrt(5))
    for r, ks in enumerate(sets):
        s = [math.fsum(qf[r, d] * kf[c, d] for d in range(5)) / math.sqrt(5) for c in ks]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        l = math.fsum(w)
        for d in range(5):
            assert abs(o[r, d] - math.fsum(w[i] * vf[c, d] for i, c in enumerate(ks)) / l) < 1e-12
        assert abs(lse[r] - (m + math.log(l))) < 1e-12


def test_constant_v_gives_constant_output():
    q, k, _ = _inputs(3, 1, 8, 256, 2, 2, 16)
    v = np.full((1, 256, 2, 16), 0.375)
    count = np.array([[[3]], [[1]]]).reshape(1, 2, 1)
    index = np.array([[[[0, 2, 3]], [[1, 0, 0]]]], np.int32).reshape(1, 2, 1, 3)
    o, _ = oracle.block_sparse(q, k, v, count, index, 8, 64)
    np.testing.assert_allclose(o, 0.375, rtol=1e-14, atol=0)   # exact up to rounding


def test_zero_q_closed_forms():
    """Q = 0: O is the mean of V over the key set and LSE = ln |K(r)| (natural log);
    with V[c, 0] = c, O[r, 0] is the mean attended position (pins which keys)."""
    B, Sq, Sk, H, D, bm, bn = 1, 6, 512, 2, 8, 2, 64
    q = np.zeros((B, Sq, H, D))
    k = bf16_to_f64(normal_bf16(4, "k", (B, Sk, H, D)))
    v = bf16_to_f64(normal_bf16(4, "v", (B, Sk, H, D)))
    v[..., 0] = np.arange(Sk)[None, :, None]
    count = np.array([[[2, 1, 3], [1, 2, 0]]], np.int32)
    index = np.array([[[[0, 5, 0], [7, 0, 0], [1, 2, 3]], [[4, 0, 0], [6, 2, 0], [0, 0, 0]]]], np.int32)
    o, lse = oracle.block_sparse(q, k, v, count, index, bm, bn, causal=True)
    for h in range(H):
        for r in range(Sq):
            i = r // bm
            keys = np.concatenate([np.arange(j * bn, (j + 1) * bn) for j in index[0, h, i, :count[0, h, i]]]
                                  ) if count[0, h, i] else np.array([], int)
            keys = keys[keys <= r + (Sk - Sq)]
            if keys.size == 0:
                assert np.all(o[0, r, h] == 0) and lse[0, h, r] == -np.inf
                continue
            np.testing.assert_allclose(o[0, r, h, 0], keys.mean(), rtol=1e-12)
            np.testing.assert_allclose(o[0, r, h, 1:], v[0, keys, h, 1:].mean(axis=0), atol=1e-12)
            np.testing.assert_allclose(lse[0, h, r], math.log(keys.size), atol=1e-12)


@pytest.mark.parametrize("Ht", ["q", "kv"])
def test_full_list_equals_dense_and_order_free(Ht):
    B, S, Hq, Hkv, D, bs = 2, 64, 4, 2, 16, 16
    q, k, v = _inputs(5, B, S, S, Hq, Hkv, D)
    H = Hq if Ht == "q" else Hkv
    nqb = nkb = S // bs
    g = rng(5, "perm")
    index = np.stack([g.permutation(nkb) for _ in range(B * H * nqb)]).reshape(B, H, nqb, nkb).astype(np.int32)
    count = np.full((B, H, nqb), nkb, np.int32)
    o, lse = oracle.block_sparse(q, k, v, count, index, bs, bs, causal=True)
    od, lsed = oracle.dense(q, k, v, causal=True)
    np.testing.assert_allclose(o, od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lsed, atol=1e-12, rtol=0)
    ref = _sdpa(bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v), causal=True)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_block_sparse_matches_sdpa_with_block_mask():
    """The block-level key sets expanded with np.kron and handed to torch SDPA as a mask."""
    B, S, H, D, bs = 1, 96, 3, 8, 32
    q, k, v = _inputs(6, B, S, S, H, H, D)
    g = rng(6, "lists")
    nqb = S // bs
    count = g.integers(1, nqb + 1, size=(B, H, nqb)).astype(np.int32)
    index = np.zeros((B, H, nqb, nqb), np.int32)
    bmask = np.zeros((B, H, nqb, nqb), bool)
    for h in range(H):
        for i in range(nqb):
            sel = g.choice(nqb, size=count[0, h, i], replace=False)
            index[0, h, i, :sel.size] = sel
            bmask[0, h, i, sel] = True
    o, lse = oracle.block_sparse(q, k, v, count, index, bs, bs)
    full = np.stack([np.kron(bmask[0, h], np.ones((bs, bs), bool)) for h in range(H)])[None]
    ref = _sdpa(bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v), mask=full)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_empty_list_is_neutral():
    q, k, v = _inputs(7, 1, 4, 128, 2, 2, 8)
    count = np.zeros((1, 2, 1), np.int32)
    index = np.zeros((1, 2, 1, 4), np.int32)
    o, lse = oracle.block_sparse(q, k, v, count, index, 4, 64)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_duplicate_entries_rejected():
    q, k, v = _inputs(7, 1, 1, 128, 1, 1, 8)
    with pytest.raises(ValueError):
        oracle.block_sparse(q, k, v, np.array([[[2]]]), np.array([[[[1, 1]]]]), 1, 64)


@pytest.mark.parametrize("case", range(38))
def test_combine_identity_disjoint_split(case):
    """FA(A u B) == Combine(FA(A), FA(B)) for disjoint block sets (workload-1 shape, seeds vary)."""
    Sk, bs, H = 1024, 64, 4
    q, k, v = _inputs(100 + case, 1, 1, Sk, H, H, 64)
    g = rng(100 + case, "split")
    nkb = Sk // bs
    na = int(g.integers(0, nkb + 1))
    a_idx = np.zeros((1, H, 1, nkb), np.int32)
    b_idx = np.zeros((1, H, 1, nkb), np.int32)
    for h in range(H):
        perm = g.permutation(nkb)
        a_idx[0, h, 0, :na] = np.sort(perm[:na])
        b_idx[0, h, 0, :nkb - na] = np.sort(perm[na:])
    ca = np.full((1, H, 1), na, np.int32)
    cb = np.full((1, H, 1), nkb - na, np.int32)
    oa, la = oracle.block_sparse(q, k, v, ca, a_idx, 1, bs)
    ob, lb = oracle.block_sparse(q, k, v, cb, b_idx, 1, bs)
    oc, lc = oracle.combine(np.stack([oa, ob]), np.stack([la, lb]))
    od, ld = oracle.dense(q, k, v)
    np.testing.assert_allclose(oc, od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lc, ld, atol=1e-12, rtol=0)


def test_combine_edge_cases():
    o = bf16_to_f64(normal_bf16(8, "o", (3, 1, 2, 2, 4)))
    lse = np.array([-np.inf, 1.5, -np.inf]).reshape(3, 1, 1, 1) * np.ones((3, 1, 2, 2))
    oc, lc = oracle.combine(o, lse)
    np.testing.assert_array_equal(oc, o[1])                      # single live partial returned unchanged
    np.testing.assert_array_equal(lc, lse[1])
    oz, lz = oracle.combine(o, np.full((3, 1, 2, 2), -np.inf))   # all empty -> (0, -inf), no NaN
    assert np.all(oz == 0) and np.all(np.isneginf(lz)) and not np.isnan(oz).any()


def test_combine_associative_and_order_free():
    o = bf16_to_f64(normal_bf16(9, "o", (4, 1, 3, 2, 8)))
    lse = bf16_to_f64(normal_bf16(9, "l", (4, 1, 2, 3))) * 3
    oc, lc = oracle.combine(o, lse)
    o01, l01 = oracle.combine(o[:2], lse[:2])
    o23, l23 = oracle.combine(o[2:], lse[2:])
    on, ln = oracle.combine(np.stack([o01, o23]), np.stack([l01, l23]))
    np.testing.assert_allclose(oc, on, atol=1e-13)
    np.testing.assert_allclose(lc, ln, atol=1e-13)
    p = [2, 0, 3, 1]
    op, lp = oracle.combine(o[p], lse[p])
    np.testing.assert_allclose(oc, op, atol=1e-13)
    np.testing.assert_allclose(lc, lp, atol=1e-13)


def test_partials_recombine_to_block_sparse():
    B, S, H, D, bs = 1, 32, 2, 8, 8
    q, k, v = _inputs(10, B, S, S, H, H, D)
    count = np.array([[[1, 2, 3, 0], [4, 1, 2, 2]]], np.int32)
    index = np.array([[[[0, 0, 0, 0], [1, 3, 0, 0], [0, 2, 3, 0], [0, 0, 0, 0]],
                       [[0, 1, 2, 3], [2, 0, 0, 0], [3, 1, 0, 0], [0, 2, 0, 0]]]], np.int32)
    op, lp = oracle.block_sparse_partials(q, k, v, count, index, bs, bs)
    assert op.shape == (4, B, S, H, D)
    oc, lc = oracle.combine(op, lp)
    o, lse = oracle.block_sparse(q, k, v, count, index, bs, bs)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(lc, lse, atol=1e-12)
    # a padding entry is the neutral partial
    assert np.all(np.isneginf(lp[3, 0, 0, :8])) and np.all(op[3, 0, :8, 0] == 0)


def test_speculative_two_pass_equals_union():
    B, Sk, Hq, Hkv, D, bs = 2, 1024, 4, 2, 32, 64
    q, k, v = _inputs(11, B, 1, Sk, Hq, Hkv, D)
    spec0 = Sk - 4 * bs
    g = rng(11, "missed")
    missed = np.stack([np.sort(g.choice(spec0 // bs, 5, replace=False)) for _ in range(B * Hkv)]
                      ).reshape(B, Hkv, 1, 5).astype(np.int32)
    mc = np.full((B, Hkv, 1), 5, np.int32)
    o, lse = oracle.speculative_sparse(q, k[:, spec0:], v[:, spec0:], k, v, mc, missed, bs, causal_spec=True)
    union = np.concatenate([missed, np.broadcast_to(np.arange(spec0 // bs, Sk // bs), (B, Hkv, 1, 4))], -1)
    ou, lu = oracle.block_sparse(q, k, v, np.full((B, Hkv, 1), 9, np.int32), union.astype(np.int32), 1, bs)
    np.testing.assert_allclose(o, ou, atol=1e-12)
    np.testing.assert_allclose(lse, lu, atol=1e-12)


def test_softcap_huge_cap_is_plain_attention():
    """tanh(x / c) * c -> x as c grows: a cap of 1e9 must reproduce plain attention (torch SDPA)."""
    q, k, v = (bf16_to_f64(normal_bf16(60, t, s)) for t, s in [("q", (2, 33, 4, 64)), ("k", (2, 47, 2, 64)),
                                                                  ("v", (2, 47, 2, 64))])
    o, lse = oracle.dense(q, k, v, causal=True, softcap=1e9)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=False, mask=np.tril(np.ones((33, 47), bool), 14)),
                               atol=1e-12)
    o0, lse0 = oracle.dense(q, k, v, causal=True)
    np.testing.assert_allclose(lse, lse0, atol=1e-12)


@pytest.mark.parametrize("scale", [0.7, 1.0 / 8.0])
def test_softcap_closed_form(scale):
    """Scores chosen through atanh so that the capped scores are known exactly: with cap c, a
    scaled score of c*atanh(1/2) becomes c/2, a score of 0 stays 0, and a very negative score
    saturates at -c.  Four keys, causal (bottom-right, Sq = Sk), so row 0 sees only key 0: a
    mask applied before the cap (tanh(-inf) = -1) would leak the other keys into it."""
    c = 3.0
    a = c * math.atanh(0.5) / scale
    q = np.zeros((1, 4, 1, 2))
    q[0, :, 0, 0] = a
    k = np.zeros((1, 4, 1, 2))
    k[0, :, 0, 0] = [1.0, 0.0, -1000.0, 0.0]
    v = np.zeros((1, 4, 1, 2))
    v[0, :, 0] = [[1.0, 0.0], [0.0, 1.0], [2.0, -2.0], [0.5, 0.25]]
    o, lse = oracle.dense(q, k, v, causal=True, scale=scale, softcap=c)
    capped = np.array([c / 2, 0.0, -c, 0.0])
    for r in range(4):
        w = np.exp(capped[:r + 1])
        np.testing.assert_allclose(o[0, r, 0], (w[:, None] * v[0, :r + 1, 0]).sum(0) / w.sum(), atol=1e-14)
        assert abs(lse[0, 0, r] - math.log(w.sum())) < 1e-14
    assert abs(lse[0, 0, 0] - c / 2) < 1e-14 and np.allclose(o[0, 0, 0], [1.0, 0.0], atol=1e-15)
