"""Pins for the oracle's gradients of block-sparse attention: torch autograd through float64
SDPA with the same key mask (GQA included), central finite differences of the oracle's own
forward, empty rows, and dense = every block listed."""
import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f64, normal_bf16, rng

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(seed, B=1, Sq=96, Sk=96, Hq=4, Hkv=2, D=16):
    q, k, v, do = (bf16_to_f64(normal_bf16(seed, t, s)) for t, s in
                   [("q", (B, Sq, Hq, D)), ("k", (B, Sk, Hkv, D)), ("v", (B, Sk, Hkv, D)), ("do", (B, Sq, Hq, D))])
    return q, k, v, do


def _lists(seed, B, H, nqb, nkb, causal, diag_off=0):
    """Random lists that always hold the block on the diagonal (so no row is empty)."""
    g = rng(seed, "bwd-lists")
    cap = nkb
    count = np.zeros((B, H, nqb), np.int32)
    index = np.zeros((B, H, nqb, cap), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                reach = min(nkb - 1, i + diag_off) if causal else nkb - 1
                others = [j for j in range(reach + 1) if j != reach and g.random() < 0.5]
                sel = np.array(sorted(set(others) | {reach}), np.int32)
                count[b, h, i] = sel.size
                index[b, h, i, :sel.size] = sel
    return count, index


@pytest.mark.parametrize("causal,Ht", [(True, "q"), (False, "kv")])
def test_matches_torch_autograd(causal, Ht):
    B, S, Hq, Hkv, D, bs = 2, 96, 4, 2, 16, 16
    q, k, v, do = _inputs(81, B, S, S, Hq, Hkv, D)
    H = Hq if Ht == "q" else Hkv
    count, index = _lists(81, B, H, S // bs, S // bs, causal)
    dq, dk, dv = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = np.zeros((B, Hq, S, S), bool)
    for b in range(B):
        for h in range(Hq):
            ht = h if Ht == "q" else h // (Hq // Hkv)
            mask[b, h] = oracle.block_mask(count[b, ht], index[b, ht], bs, bs, S, S)
            if causal:
                mask[b, h] &= np.tril(np.ones((S, S), bool))
    o = torch.nn.functional.scaled_dot_product_attention(tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3),
                                                         tv.permute(0, 2, 1, 3), attn_mask=torch.from_numpy(mask),
                                                         enable_gqa=True).permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_finite_differences_of_the_forward():
    """Central differences of L = sum(O * dO) through the oracle's forward, at sampled entries."""
    B, S, Hq, Hkv, D, bs = 1, 32, 2, 1, 8, 8
    q, k, v, do = _inputs(82, B, S, S, Hq, Hkv, D)
    count, index = _lists(82, B, Hq, S // bs, S // bs, True)
    dq, dk, dv = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, True)

    def loss(qq, kk, vv):
        o, _ = oracle.block_sparse(qq, kk, vv, count, index, bs, bs, causal=True)
        return float((o * do).sum())

    g = rng(82, "fd")
    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(g.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            lp = loss(*(xp if a is x else a for a in args))
            lm = loss(*(xm if a is x else a for a in args))
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-7, (name, idx)


def test_empty_rows_and_dense():
    B, S, Hq, Hkv, D, bs = 1, 64, 2, 2, 16, 16
    q, k, v, do = _inputs(83, B, S, S, Hq, Hkv, D)
    nb = S // bs
    count = np.full((B, Hq, nb), nb, np.int32)
    index = np.broadcast_to(np.arange(nb, dtype=np.int32), (B, Hq, nb, nb)).copy()
    dense = oracle.block_sparse_bwd(q, k, v, do, causal=True)
    listed = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, True)
    for a, b in zip(dense, listed):
        np.testing.assert_allclose(a, b, atol=1e-13)
    count[0, 1, 2] = 0                                    # query block 2 of head 1: no keys
    dq, dk, dv = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, True)
    assert np.all(dq[0, 2 * bs:3 * bs, 1] == 0)
    # the emptied rows no longer feed dK / dV of head 1: removing their dO changes nothing
    do2 = do.copy()
    do2[0, 2 * bs:3 * bs, 1] = 0
    for a, b in zip((dk, dv), oracle.block_sparse_bwd(q, k, v, do2, count, index, bs, bs, True)[1:]):
        np.testing.assert_allclose(a, b, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_softcap_matches_torch_autograd(causal):
    """Softcapped scores c tanh(x / c) before the mask and softmax, differentiated by torch."""
    B, S, Hq, Hkv, D, bs, cap = 1, 64, 4, 2, 16, 16, 2.5
    q, k, v, do = _inputs(84, B, S, S, Hq, Hkv, D)
    count, index = _lists(84, B, Hq, S // bs, S // bs, causal)
    dq, dk, dv = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, causal, softcap=cap)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    scale = 1.0 / np.sqrt(D)
    G = Hq // Hkv
    loss = 0.0
    for h in range(Hq):
        mask = oracle.block_mask(count[0, h], index[0, h], bs, bs, S, S)
        if causal:
            mask &= np.tril(np.ones((S, S), bool))
        x = scale * tq[0, :, h] @ tk[0, :, h // G].T
        x = cap * torch.tanh(x / cap)
        x = x.masked_fill(~torch.from_numpy(mask), float("-inf"))
        o = torch.softmax(x, dim=1) @ tv[0, :, h // G]
        loss = loss + (o * torch.from_numpy(do[0, :, h])).sum()
    loss.backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_softcap_finite_differences():
    B, S, Hq, Hkv, D, bs, cap = 1, 32, 2, 1, 8, 8, 1.5
    q, k, v, do = _inputs(85, B, S, S, Hq, Hkv, D)
    count, index = _lists(85, B, Hq, S // bs, S // bs, True)
    dq, dk, dv = oracle.block_sparse_bwd(q, k, v, do, count, index, bs, bs, True, softcap=cap)

    def loss(qq, kk, vv):
        o, _ = oracle.block_sparse(qq, kk, vv, count, index, bs, bs, causal=True, softcap=cap)
        return float((o * do).sum())

    g = rng(85, "fd")
    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(g.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            lp = loss(*(xp if a is x else a for a in (q, k, v)))
            lm = loss(*(xm if a is x else a for a in (q, k, v)))
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-7, (name, idx)
