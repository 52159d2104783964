"""Pins for the oracle's selected attention (top-k key blocks per query token): torch SDPA with
an independently built mask, dense causal when every reachable block is selected, the combine
identity over a split selection, empty selections, row spot checks and the fixed-length form."""
import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f64
from synth.workloads import selected_prefill

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _small(seed=61, seqlens=(300, 130), Hq=4, Hkv=2, D=16, block=16, topk=5):
    return selected_prefill(seed=seed, seqlens=seqlens, Hq=Hq, Hkv=Hkv, D=D, block=block, topk=topk)


def _sdpa_seq(w, b, h, mask):
    cu = w["cu_seqlens"]
    a, e = int(cu[b]), int(cu[b + 1])
    G = w["Hq"] // w["Hkv"]
    q = torch.from_numpy(bf16_to_f64(w["q"][a:e, h]))[None, None]
    k = torch.from_numpy(bf16_to_f64(w["k"][a:e, h // G]))[None, None]
    v = torch.from_numpy(bf16_to_f64(w["v"][a:e, h // G]))[None, None]
    am = torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am)[0, 0].numpy()


def test_matches_sdpa_with_block_level_mask():
    w = _small()
    o, lse = oracle.selected(w["q"], w["k"], w["v"], w["sel"], w["block"], w["cu_seqlens"], w["cu_seqlens"])
    cu, bs = w["cu_seqlens"], w["block"]
    G = w["Hq"] // w["Hkv"]
    for b in range(2):
        a, e = int(cu[b]), int(cu[b + 1])
        n = e - a
        nkb = -(-n // bs)
        for h in range(w["Hq"]):
            sel = w["sel"][a:e, h // G]
            blk = np.zeros((n, nkb), bool)
            rr, cc = np.nonzero(sel >= 0)
            blk[rr, sel[rr, cc]] = True
            mask = np.repeat(blk, bs, axis=1)[:, :n] & np.tril(np.ones((n, n), bool))
            np.testing.assert_allclose(o[a:e, h], _sdpa_seq(w, b, h, mask), atol=1e-12)


def test_every_reachable_block_is_dense_causal():
    w = _small(topk=64)
    assert (w["sel"] >= 0).sum(axis=-1).max() <= 64
    o, lse = oracle.selected(w["q"], w["k"], w["v"], w["sel"], w["block"], w["cu_seqlens"], w["cu_seqlens"])
    cu = w["cu_seqlens"]
    for b in range(2):
        a, e = int(cu[b]), int(cu[b + 1])
        n = e - a
        for h in (0, 3):
            np.testing.assert_allclose(o[a:e, h], _sdpa_seq(w, b, h, np.tril(np.ones((n, n), bool))), atol=1e-12)


def test_combine_of_split_selection():
    """Slots 0..2 and 3..4 of every token are disjoint block sets: attention over each, merged
    with the log-sum-exp combine, equals attention over the union."""
    w = _small()
    cu = w["cu_seqlens"]
    sa, sb = w["sel"].copy(), w["sel"].copy()
    sa[..., 3:] = -1
    sb[..., :3] = -1
    oa, la = oracle.selected(w["q"], w["k"], w["v"], sa, w["block"], cu, cu)
    ob, lb = oracle.selected(w["q"], w["k"], w["v"], sb, w["block"], cu, cu)
    o, lse = oracle.selected(w["q"], w["k"], w["v"], w["sel"], w["block"], cu, cu)
    # combine works on [P, B, Sq, H, D] / [P, B, H, Sq]: one batch of all tokens
    oc, lc = oracle.combine(np.stack([oa, ob])[:, None], np.stack([la, lb])[:, None])
    np.testing.assert_allclose(oc[0], o, atol=1e-12)
    np.testing.assert_allclose(lc[0], lse, atol=1e-12)


def test_empty_selection_and_rows_and_fixed_length():
    w = _small()
    cu = w["cu_seqlens"]
    sel = w["sel"].copy()
    sel[5] = -1
    o, lse = oracle.selected(w["q"], w["k"], w["v"], sel, w["block"], cu, cu)
    assert np.all(o[5] == 0) and np.isneginf(lse[:, 5]).all()
    rows = np.array([0, 17, 129])
    for b, h in [(0, 1), (1, 3)]:
        orow, lrow = oracle.selected_rows(w["q"], w["k"], w["v"], sel, w["block"], cu, cu, b, h, rows)
        a = int(cu[b])
        np.testing.assert_allclose(orow, o[a + rows, h], atol=1e-12)
        np.testing.assert_allclose(lrow, lse[h, a + rows], atol=1e-12)
    # two sequences of equal length as a fixed-length batch
    w2 = _small(seqlens=(160, 160))
    c2 = w2["cu_seqlens"]
    ov, lv = oracle.selected(w2["q"], w2["k"], w2["v"], w2["sel"], w2["block"], c2, c2)
    of, lf = oracle.selected(w2["q"].reshape(2, 160, 4, 16), w2["k"].reshape(2, 160, 2, 16),
                             w2["v"].reshape(2, 160, 2, 16), w2["sel"].reshape(2, 160, 2, 5), w2["block"])
    np.testing.assert_allclose(of.reshape(320, 4, 16), ov, atol=1e-15)
    np.testing.assert_allclose(lf.transpose(1, 0, 2).reshape(4, 320), lv, atol=1e-15)


def test_repeated_block_rejected():
    w = _small()
    sel = w["sel"].copy()
    sel[40, 0, :2] = 0
    with pytest.raises(ValueError):
        oracle.selected(w["q"], w["k"], w["v"], sel, w["block"], w["cu_seqlens"], w["cu_seqlens"])
