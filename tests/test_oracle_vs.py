"""Pins for the oracle's vertical-slash conversion (invariants against a brute-force bitmap of
the exact pattern) and for attention over the converted metadata (special cases that reduce to
dense or block-diagonal causal attention, and a closed form)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f64, normal_bf16, power_law_unique, rng
from synth.workloads import vs_varlen_prefill

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _exact_pattern(q_len, kv_len, vert, slash, r0, r1):
    """Bitmap [rows, kv_len] of the raw pattern: (r, r + d - s) for each slash s, (r, v) for each
    vertical v that row r can see (v <= r + d)."""
    d = kv_len - q_len
    bm = np.zeros((r1 - r0, kv_len), bool)
    for i, r in enumerate(range(r0, r1)):
        for s in slash:
            c = r + d - int(s)
            if 0 <= c < kv_len:
                bm[i, c] = True
        for v in vert:
            if int(v) <= r + d:
                bm[i, int(v)] = True
    return bm


@pytest.mark.parametrize("seed", range(12))
def test_conversion_invariants(seed):
    g = rng(seed, "vs-inv")
    q_len = int(g.integers(1, 300))
    kv_len = q_len + int(g.integers(0, 3)) * int(g.integers(0, 50))
    bM = int(g.choice([8, 16, 32]))
    bN = int(g.choice([bM, 2 * bM]))
    nv, ns = int(g.integers(0, 40)), int(g.integers(1, 40))
    vert = np.sort(power_law_unique(g, kv_len, nv, force_zero=nv > 0))[:nv]
    slash = np.sort(power_law_unique(g, kv_len, ns))[::-1]
    context = q_len + int(g.integers(0, 100))
    R = -(-context // bM)
    for m in range(R):
        w, c = oracle.vs_convert_item(q_len, kv_len, vert, slash, m, bM, bN)
        r0 = m * bM
        if r0 >= q_len:
            assert w == [] and c == []
            continue
        r1 = min(r0 + bM, q_len)
        d = kv_len - q_len
        assert len(w) <= len(slash) and len(c) <= len(vert)
        assert all(w[i] + bN <= w[i + 1] for i in range(len(w) - 1))       # disjoint, ascending
        assert all(x >= 0 for x in w)
        assert all(c[i] < c[i + 1] for i in range(len(c) - 1))             # ascending, unique
        assert set(c) <= set(int(x) for x in vert)
        assert all(x <= r1 - 1 + d for x in c)                             # visible to the block
        assert not any(wi <= x < wi + bN for x in c for wi in w)           # outside every window
        exact = _exact_pattern(q_len, kv_len, vert, slash, r0, r1)
        cover = np.zeros(kv_len, bool)
        for wi in w:
            cover[wi:wi + bN] = True
        cover[c] = True
        assert not (exact & ~cover[None, :]).any()                          # pattern covered
        starts_on_pattern = exact.any(axis=0)
        assert all(starts_on_pattern[wi] for wi in w)                       # each window starts on it


def _run_vs(w, vert, slash, causal=True):
    cu = w["cu_seqlens"]
    bc, bo, cc, ci = oracle.vs_convert(w["seqlens"], w["seqlens"], vert, slash, w["context_size"],
                                       w["block_M"], w["block_N"])
    return oracle.vs_attention(w["q"], w["k"], w["v"], bc, bo, cc, ci, cu, cu, w["block_M"], w["block_N"], causal)


def _sdpa_seq(w, b, mask):
    cu = w["cu_seqlens"]
    a, e = cu[b], cu[b + 1]
    t = [torch.from_numpy(bf16_to_f64(x[a:e])).permute(1, 0, 2)[None] for x in (w["q"], w["k"], w["v"])]
    o = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=torch.from_numpy(mask))
    return o[0].permute(1, 0, 2).numpy()


def _small_vs():
    return vs_varlen_prefill(seed=31, seqlens=(96, 40), H=2, D=16, nnz_v=4, nnz_s=4, block=16,
                             context_size=112)


def test_all_slashes_is_dense_causal():
    """Every diagonal offset 0..n-1 listed: the converted pattern is dense causal attention."""
    w = _small_vs()
    H = 2
    for b in range(2):
        n = int(w["seqlens"][b])
        sl = w["seqlens"][b:b + 1]
        slash = np.broadcast_to(np.arange(n)[::-1], (1, H, n)).astype(np.int32)
        bc, bo, cc, ci = oracle.vs_convert(sl, sl, np.zeros((1, H, 0), np.int32), slash, w["context_size"], 16, 16)
        cu = np.array([0, n], np.int32)
        a = int(w["cu_seqlens"][b])
        o, _ = oracle.vs_attention(w["q"][a:a + n], w["k"][a:a + n], w["v"][a:a + n], bc, bo, cc, ci, cu, cu, 16, 16)
        np.testing.assert_allclose(o, _sdpa_seq(w, b, np.tril(np.ones((n, n), bool))), atol=1e-12)


def test_main_diagonal_only_is_block_diagonal_causal():
    w = _small_vs()
    B, H = 2, 2
    o, _ = _run_vs(w, np.zeros((B, H, 0), np.int32), np.zeros((B, H, 1), np.int32))
    for b in range(B):
        n = int(w["seqlens"][b])
        r = np.arange(n)
        mask = (r[None, :] <= r[:, None]) & (r[None, :] >= (r[:, None] // 16) * 16)
        a = int(w["cu_seqlens"][b])
        np.testing.assert_allclose(o[a:a + n], _sdpa_seq(w, b, mask), atol=1e-12)


def test_all_verticals_is_dense_causal():
    w = _small_vs()
    B, H = 2, 2
    vert = np.zeros((B, H, 96), np.int32)
    for b in range(B):
        n = int(w["seqlens"][b])
        vert[b, :, :] = np.minimum(np.arange(96), n - 1)
    for b in range(B):
        n = int(w["seqlens"][b])
        cu = np.array([0, n], np.int32)
        sl = w["seqlens"][b:b + 1]
        # slash offset n + 5 lies beyond every row: contributes no window
        bc, bo, cc, ci = oracle.vs_convert(sl, sl, vert[b:b + 1, :, :n], np.full((1, H, 1), n + 5, np.int32),
                                           w["context_size"], 16, 16)
        assert bc.sum() == 0
        a = int(w["cu_seqlens"][b])
        o, _ = oracle.vs_attention(w["q"][a:a + n], w["k"][a:a + n], w["v"][a:a + n], bc, bo, cc, ci, cu, cu, 16, 16)
        np.testing.assert_allclose(o, _sdpa_seq(w, b, np.tril(np.ones((n, n), bool))), atol=1e-12)


def test_zero_q_lse_counts_keys():
    w = _small_vs()
    w["q"] = np.zeros_like(w["q"])
    bc, bo, cc, ci = oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], w["context_size"], 16, 16)
    o, lse = oracle.vs_attention(w["q"], w["k"], w["v"], bc, bo, cc, ci, w["cu_seqlens"], w["cu_seqlens"], 16, 16)
    for b in range(2):
        n = int(w["seqlens"][b])
        a = int(w["cu_seqlens"][b])
        for h in range(2):
            for r in range(n):
                m = r // 16
                keys = set()
                for x in bo[b, h, m, :bc[b, h, m]]:
                    keys.update(range(x, min(n, x + 16)))
                keys.update(ci[b, h, m, :cc[b, h, m]].tolist())
                keys = [c for c in keys if c <= r]
                assert abs(lse[h, a + r] - math.log(len(keys))) < 1e-12


def test_rows_match_full_and_generator_shapes():
    w = vs_varlen_prefill(seed=32, seqlens=(200, 120), H=2, D=16, nnz_v=12, nnz_s=20, block=16, context_size=224)
    assert w["vertical"].shape == (2, 2, 12) and w["slash"].shape == (2, 2, 20)
    assert (np.diff(w["vertical"], axis=-1) > 0).all() and (np.diff(w["slash"], axis=-1) < 0).all()
    assert (w["vertical"][..., 0] == 0).all() and (w["slash"][..., -1] == 0).all()
    bc, bo, cc, ci = oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], 224, 16, 16)
    assert bc.shape == (2, 2, 14) and (bc[1, :, 8:] == 0).all()
    o, lse = oracle.vs_attention(w["q"], w["k"], w["v"], bc, bo, cc, ci, w["cu_seqlens"], w["cu_seqlens"], 16, 16)
    for b, h, m in [(0, 1, 12), (1, 0, 7), (0, 0, 0)]:
        rows = np.arange(m * 16, min(int(w["seqlens"][b]), m * 16 + 16))
        orow, lrow = oracle.vs_attention_rows(w["q"], w["k"], w["v"], b, h, rows, bo[b, h, m, :bc[b, h, m]],
                                              ci[b, h, m, :cc[b, h, m]], w["cu_seqlens"], w["cu_seqlens"], 16)
        a = int(w["cu_seqlens"][b])
        np.testing.assert_allclose(orow, o[a + rows, h], atol=1e-12)
        np.testing.assert_allclose(lrow, lse[h, a + rows], atol=1e-12)


def test_power_law_generator():
    g = rng(7, "pl")
    x = power_law_unique(g, 65536, 2000)
    assert x.size == 2000 and np.unique(x).size == 2000 and 0 in x and x.max() < 65536
    assert np.median(x) < 5000                    # heavy head: most mass near 0


@pytest.mark.parametrize("seed", range(4))
def test_mergehead_ignores_entries_past_the_counts(seed):
    """Merged-head conversion: entries past a head's count must not matter.  Fill them with
    values that would change the result if read (vertical 0..n-1, slash offset 0), and compare
    with the plain conversion of rows whose tails hold inert values instead (a vertical index past
    every key, a slash offset past every row: neither can reach a key)."""
    g = rng(seed, "vs-mergehead")
    w = vs_varlen_prefill(seed=40 + seed, seqlens=(190, 77), H=3, D=16, nnz_v=14, nnz_s=18, block=16,
                          context_size=192)
    B, H = 2, 3
    vc = g.integers(0, 15, size=H).astype(np.int32)
    sc = g.integers(0, 19, size=H).astype(np.int32)
    vc[0], sc[1] = 14, 0  # a full count and an empty one
    vert, slash = w["vertical"].copy(), w["slash"].copy()
    inert_v, inert_s = vert.copy(), slash.copy()
    for h in range(H):
        vert[:, h, vc[h]:] = np.arange(14 - vc[h])
        slash[:, h, sc[h]:] = 0
        inert_v[:, h, vc[h]:] = 10_000
        inert_s[:, h, sc[h]:] = 10_000
    got = oracle.vs_convert_mergehead(w["seqlens"], w["seqlens"], vert, slash, vc, sc, 192, 16, 16)
    want = oracle.vs_convert(w["seqlens"], w["seqlens"], inert_v, inert_s, 192, 16, 16)
    for x, y in zip(got, want):
        assert np.array_equal(x, y)
    # the planted tails do change the plain conversion wherever a count is short
    planted = oracle.vs_convert(w["seqlens"], w["seqlens"], vert, slash, 192, 16, 16)
    assert not all(np.array_equal(x, y) for x, y in zip(planted, want))
    # counts at least NNZ (clamped) give the plain conversion of the full rows
    full = oracle.vs_convert_mergehead(w["seqlens"], w["seqlens"], w["vertical"], w["slash"],
                                       np.full(H, 99, np.int32), np.full(H, 18, np.int32), 192, 16, 16)
    for x, y in zip(full, oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], 192, 16, 16)):
        assert np.array_equal(x, y)
