"""GPU parity for vertical-slash conversion (bit-exact counts and valid prefixes) and varlen
attention over the converted metadata, at small size (everything) and full size (every
conversion item; every row of sampled query blocks)."""
import os

import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import normal_bf16
from synth.workloads import vs_varlen_prefill
from tests.golden.make_full_size import vs_digest
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_size.npz")

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _convert(w):
    sl = dev_i32(w["seqlens"])
    return bsa.vs_convert_indexes(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), w["context_size"],
                                  w["block_M"], w["block_N"])


def _check_items(gpu, w, items, host_arrays=False):
    bc, bo, cc, ci = gpu if host_arrays else (x.cpu().numpy() for x in gpu)
    for b, h, m in items:
        L = int(w["seqlens"][b])
        wins, cols = oracle.vs_convert_item(L, L, w["vertical"][b, h], w["slash"][b, h], m, w["block_M"], w["block_N"])
        assert bc[b, h, m] == len(wins) and cc[b, h, m] == len(cols), (b, h, m)
        assert np.array_equal(bo[b, h, m, :len(wins)], wins), (b, h, m)
        assert np.array_equal(ci[b, h, m, :len(cols)], cols), (b, h, m)


@pytest.mark.parametrize("seqlens,ctx", [((300, 170), 320), ((64, 1), 64), ((1000, 999, 5), 1024)])
def test_convert_small_exact(seqlens, ctx):
    say("vs convert small", seqlens)
    w = vs_varlen_prefill(seed=51, seqlens=seqlens, H=3, D=128, nnz_v=20, nnz_s=30, block=64, context_size=ctx)
    gpu = _convert(w)
    R = -(-ctx // 64)
    _check_items(gpu, w, [(b, h, m) for b in range(len(seqlens)) for h in range(3) for m in range(R)])


@pytest.mark.parametrize("bm,bn", [(64, 64), (64, 128)])
def test_convert_mergehead_exact(bm, bn):
    """Per-head counts: heads with a full count, an empty count, a count past NNZ (clamped) and
    partial counts; bit-exact against the oracle on every query block."""
    say("vs convert mergehead", bm, bn)
    w = vs_varlen_prefill(seed=54, seqlens=(700, 300, 64), H=5, D=128, nnz_v=40, nnz_s=60, block=64,
                          context_size=768)
    vc = np.array([40, 0, 17, 99, 3], np.int32)
    sc = np.array([0, 60, 25, 1, 70], np.int32)
    sl = dev_i32(w["seqlens"])
    gpu = bsa.vs_convert_indexes_mergehead(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), dev_i32(vc),
                                           dev_i32(sc), 768, bm, bn)
    bc, bo, cc, ci = (x.cpu().numpy() for x in gpu)
    rb, rbo, rcc, rci = oracle.vs_convert_mergehead(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], vc, sc,
                                                    768, bm, bn)
    assert np.array_equal(bc, rb) and np.array_equal(cc, rcc)
    for b, h, m in np.ndindex(*rb.shape):
        assert np.array_equal(bo[b, h, m, :rb[b, h, m]], rbo[b, h, m, :rb[b, h, m]]), (b, h, m)
        assert np.array_equal(ci[b, h, m, :rcc[b, h, m]], rci[b, h, m, :rcc[b, h, m]]), (b, h, m)


@pytest.mark.parametrize("bm,bn", [(64, 64), (64, 128), (128, 128)])
def test_attention_small_varlen(bm, bn):
    """Both tile sizes of the prefill kernel (64-row tiles with 32-key chunks, 128-row tiles
    with 64-key chunks) and windows spanning one or two chunks."""
    w = vs_varlen_prefill(seed=52, seqlens=(700, 300, 64), H=4, D=128, nnz_v=40, nnz_s=60, block=64,
                          context_size=768)
    say("vs attention small varlen", bm, bn)
    sl = dev_i32(w["seqlens"])
    bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), 768, bm, bn)
    pat = bsa.VSPattern(bc, bo, cc, ci, bm, bn)
    cu = dev_i32(w["cu_seqlens"])
    o, lse = bsa.bsa_fwd(dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"]), pat, causal=True,
                         out_dtype=torch.float32, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=700,
                         max_seqlen_k=700)
    rb, rbo, rcc, rci = oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], 768, bm, bn)
    o_ref, lse_ref = oracle.vs_attention(w["q"], w["k"], w["v"], rb, rbo, rcc, rci, w["cu_seqlens"],
                                         w["cu_seqlens"], bm, bn)
    check_o(host(o), o_ref, "vs attention")
    check_lse(host(lse), lse_ref, "vs attention lse")


@pytest.mark.parametrize("causal", [True, False])
def test_attention_fixed_length_gqa(causal):
    """Fixed-length (batch, seqlen, heads, dim) inputs as the pages' sparse_attn_func takes them,
    GQA (two query heads per key/value head), with and without the causal mask; the metadata
    comes from the causal conversion either way."""
    B, S, H, Hkv = 2, 640, 4, 2
    w = vs_varlen_prefill(seed=53, seqlens=(S, S), H=H, D=128, nnz_v=30, nnz_s=50, block=64, context_size=S)
    say("vs attention fixed length, causal =", causal)
    sl = dev_i32(w["seqlens"])
    bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), S, 64, 64)
    q4 = w["q"].reshape(B, S, H, 128)
    k4 = w["k"].reshape(B, S, H, 128)[:, :, :Hkv]
    v4 = w["v"].reshape(B, S, H, 128)[:, :, :Hkv]
    o, lse = bsa.bsa_fwd(dev_bf16(q4), dev_bf16(k4), dev_bf16(v4), bsa.VSPattern(bc, bo, cc, ci, 64, 64),
                         causal=causal, out_dtype=torch.float32)
    rb, rbo, rcc, rci = oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], S, 64, 64)
    o_ref, lse_ref = oracle.vs_attention(w["q"], k4.reshape(B * S, Hkv, 128), v4.reshape(B * S, Hkv, 128),
                                         rb, rbo, rcc, rci, w["cu_seqlens"], w["cu_seqlens"], 64, 64,
                                         causal=causal)
    check_o(host(o).reshape(B * S, H, 128), o_ref, "vs fixed length")
    # varlen LSE is [H, total]; fixed-length LSE is [B, H, S]
    check_lse(host(lse).transpose(1, 0, 2).reshape(H, B * S), lse_ref, "vs fixed length lse")


@pytest.mark.parametrize("bn", [64, 128])
def test_attention_varlen_lists_per_kv_head(bn):
    """GQA with the converted metadata given per kv head (two query heads share each list), on
    packed sequences whose block counts are odd (a query block without a neighbour to pair
    with).  The oracle takes the metadata per query head, so each kv head's lists are repeated
    for its query heads on the host."""
    Hq, Hkv = 4, 2
    w = vs_varlen_prefill(seed=54, seqlens=(704, 320, 64), H=Hkv, D=128, nnz_v=40, nnz_s=60, block=64,
                          context_size=768)
    say("vs attention varlen, lists per kv head", bn)
    q = normal_bf16(54, "q gqa", (w["q"].shape[0], Hq, 128))
    sl = dev_i32(w["seqlens"])
    bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), 768, 64, bn)
    cu = dev_i32(w["cu_seqlens"])
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(w["k"]), dev_bf16(w["v"]), bsa.VSPattern(bc, bo, cc, ci, 64, bn),
                         causal=True, out_dtype=torch.float32, cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=704,
                         max_seqlen_k=704)
    rb, rbo, rcc, rci = oracle.vs_convert(w["seqlens"], w["seqlens"], w["vertical"], w["slash"], 768, 64, bn)
    rep = [np.repeat(x, Hq // Hkv, axis=1) for x in (rb, rbo, rcc, rci)]
    o_ref, lse_ref = oracle.vs_attention(q, w["k"], w["v"], *rep, w["cu_seqlens"], w["cu_seqlens"], 64, bn)
    check_o(host(o), o_ref, "vs attention, lists per kv head")
    check_lse(host(lse), lse_ref, "vs attention lse, lists per kv head")


@pytest.fixture(scope="module")
def cfg5():
    say("generating vertical-slash varlen workload (seqlens 65536 + 32768, H=32)")
    w = vs_varlen_prefill()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


def test_full_size_convert_every_item(cfg5):
    """All 65,536 (sequence, head, query block) items of the conversion, bit-exact: each
    (sequence, head) row's counts and valid prefixes are digested and compared with the oracle's
    (stored by tests/golden/make_full_size.py); a differing row is then walked item by item."""
    w = cfg5
    gold = np.load(GOLDEN, allow_pickle=False)["vs_sha"]
    say("vs convert full size, every item")
    bc, bo, cc, ci = (x.cpu().numpy() for x in _convert(w))
    assert bc.shape == (2, 32, 1024) and bo.shape == (2, 32, 1024, 2000) and ci.shape == (2, 32, 1024, 1000)
    bad = [(b, h) for b in range(2) for h in range(32) if vs_digest(bc[b, h], bo[b, h], cc[b, h], ci[b, h]).encode()
           != gold[b, h]]
    if bad:
        b, h = bad[0]
        _check_items((bc, bo, cc, ci), w, [(b, h, m) for m in range(1024)], host_arrays=True)
        raise AssertionError(f"conversion digests differ for (sequence, head) rows {bad}")
    assert (bc[1, :, 512:] == 0).all() and (cc[1, :, 512:] == 0).all()
    print(f"[parity] vs conversion full size: 65536 items bit-exact, {int(bc.sum())} windows, "
          f"{int(cc.sum())} columns", flush=True)


def test_full_size_attention(cfg5):
    """Every row of 12 query blocks of the varlen attention over the converted metadata: both
    sequences, first, middle and last blocks, several heads."""
    w = cfg5
    say("vs attention full size")
    bc, bo, cc, ci = _convert(w)
    pat = bsa.VSPattern(bc, bo, cc, ci, 64, 64)
    cu = dev_i32(w["cu_seqlens"])
    o, lse = bsa.bsa_fwd(w["dq"], w["dk"], w["dv"], pat, causal=True, out_dtype=torch.float32, cu_seqlens_q=cu,
                         cu_seqlens_k=cu, max_seqlen_q=65536, max_seqlen_k=65536)
    oh, lh = host(o), host(lse)
    for b, h, m in [(0, 3, 1023), (1, 30, 511), (0, 11, 400), (1, 0, 0), (0, 20, 7), (0, 31, 0), (1, 16, 256),
                    (0, 0, 1022), (1, 9, 510), (0, 25, 640), (1, 4, 100), (0, 14, 900)]:
        L = int(w["seqlens"][b])
        rows = np.arange(m * 64, min(L, m * 64 + 64))
        wins, cols = oracle.vs_convert_item(L, L, w["vertical"][b, h], w["slash"][b, h], m, 64, 64)
        o_ref, lse_ref = oracle.vs_attention_rows(w["q"], w["k"], w["v"], b, h, rows, wins, cols, w["cu_seqlens"],
                                                  w["cu_seqlens"], 64)
        a = int(w["cu_seqlens"][b])
        check_o(oh[a + rows, h], o_ref, f"vs full b={b} h={h} m={m}")
        check_lse(lh[h, a + rows], lse_ref, f"vs full lse b={b} h={h} m={m}")


def test_full_size_attention_every_block_of_a_head(cfg5):
    """Every query block of one head of each sequence (1,536 blocks: both blocks of every pair
    the kernel takes together), two rows each: a random one and the block's last row, whose
    causal limit reaches furthest."""
    w = cfg5
    say("vs attention full size, every query block of two heads")
    bc, bo, cc, ci = _convert(w)
    pat = bsa.VSPattern(bc, bo, cc, ci, 64, 64)
    cu = dev_i32(w["cu_seqlens"])
    o, lse = bsa.bsa_fwd(w["dq"], w["dk"], w["dv"], pat, causal=True, out_dtype=torch.float32, cu_seqlens_q=cu,
                         cu_seqlens_k=cu, max_seqlen_q=65536, max_seqlen_k=65536)
    oh, lh = host(o), host(lse)
    g = np.random.default_rng(1005)
    worst_o = worst_l = 0.0
    for b, h in [(0, 5), (1, 22)]:
        L = int(w["seqlens"][b])
        a = int(w["cu_seqlens"][b])
        o_ref = np.zeros((L // 64, 2, 128))
        l_ref = np.zeros((L // 64, 2))
        rows = np.zeros((L // 64, 2), np.int64)
        for m in range(L // 64):
            rows[m] = (m * 64 + int(g.integers(0, 63)), m * 64 + 63)
            wins, cols = oracle.vs_convert_item(L, L, w["vertical"][b, h], w["slash"][b, h], m, 64, 64)
            o_ref[m], l_ref[m] = oracle.vs_attention_rows(w["q"], w["k"], w["v"], b, h, rows[m], wins, cols,
                                                           w["cu_seqlens"], w["cu_seqlens"], 64)
        worst_o = max(worst_o, check_o(oh[a + rows, h], o_ref, f"vs full b={b} h={h} every block"))
        worst_l = max(worst_l, check_lse(lh[h, a + rows], l_ref, f"vs full lse b={b} h={h} every block"))
    print(f"[parity] vs attention, every query block of two heads: max |dO| {worst_o:.3e}, "
          f"max |dLSE| {worst_l:.3e}", flush=True)
