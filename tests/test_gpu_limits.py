"""GPU parity where the kernels' LDS staging overflows and the tails are read from global
memory: block lists of more than 256 entries (prefill and a decode split of more than 256
entries), vertical-slash blocks with more than 768 gathered columns or more than 256 windows (the
windows each block of a query-block pair stages), and conversions with many indices: more slash
indices per head than the window walk stages in LDS (16,384) and more windows per query block
than the column test stages (4,096).  Expected values come from the oracle."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import normal_bf16, rng
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def test_prefill_list_longer_than_staging():
    B, Sq, Sk, Hq, Hkv, cap = 1, 256, 20480, 2, 1, 300
    say("prefill list of 300 entries")
    q, k, v = (normal_bf16(101, n, s) for n, s in (("q", (B, Sq, Hq, 128)), ("k", (B, Sk, Hkv, 128)),
                                                    ("v", (B, Sk, Hkv, 128))))
    g = rng(101, "long list")
    nqb, nkb = Sq // 128, Sk // 64
    count = np.full((B, Hq, nqb), cap, np.int32)
    index = np.stack([np.stack([g.choice(nkb, cap, replace=False) for _ in range(nqb)]) for _ in range(Hq)])[None]
    index = index.astype(np.int32)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), 128, 64)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, count, index, 128, 64)
    check_o(host(o), o_ref, "prefill 300-entry lists")
    check_lse(host(lse), lse_ref, "prefill 300-entry lists lse")


def test_decode_partial_longer_than_staging():
    """bsa_fwd_partials with 300 entries per partial on the decode path: one split walks 300
    list entries, past the 256 it stages in LDS."""
    B, Sk, Hq, Hkv, cap = 2, 24576, 8, 2, 320
    say("decode partials of 300 entries")
    q, k, v = (normal_bf16(102, n, s) for n, s in (("q", (B, 1, Hq, 128)), ("k", (B, Sk, Hkv, 128)),
                                                    ("v", (B, Sk, Hkv, 128))))
    g = rng(102, "decode long list")
    nkb = Sk // 64
    count = np.full((B, Hkv, 1), cap, np.int32)
    index = np.stack([np.stack([g.choice(nkb, cap, replace=False)[None] for _ in range(Hkv)]) for _ in range(B)])
    index = index.astype(np.int32)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), 128, 64)
    op, lp = bsa.bsa_fwd_partials(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, 300)
    assert op.shape[0] == 2
    o, lse = bsa.bsa_combine(op, lp, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, count, index, 128, 64)
    check_o(host(o), o_ref, "decode 300-entry partial")
    check_lse(host(lse), lse_ref, "decode 300-entry partial lse")


def _vs_inputs(seed, L, H, nnz_v, nnz_s):
    g = rng(seed, "vs limits")
    vert = np.stack([np.sort(g.choice(L, nnz_v, replace=False)) for _ in range(H)])[None].astype(np.int32)
    slash = np.stack([np.sort(g.choice(L, nnz_s, replace=False))[::-1] for _ in range(H)])[None].astype(np.int32)
    return vert, slash


@pytest.mark.parametrize("blk", [64, 128])
def test_vs_columns_longer_than_staging(blk):
    """More gathered columns per query block than the kernels stage in LDS (768): the rest are
    read from memory.  64-row tiles (64-key windows) and 128-row tiles (128-key windows)."""
    L, H = 4096, 2
    say(f"vertical-slash with more than 768 columns per block, {blk}-row blocks")
    vert, slash = _vs_inputs(103, L, H, 1500, 10)
    q, k, v = (normal_bf16(103, n, (L, H, 128)) for n in ("q", "k", "v"))
    sl = dev_i32([L])
    bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, dev_i32(vert), dev_i32(slash), L, blk, blk)
    assert int(host(cc).max()) > 768
    cu = np.array([0, L], np.int32)
    pat = bsa.VSPattern(bc, bo, cc, ci, blk, blk)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, causal=True, out_dtype=torch.float32,
                         cu_seqlens_q=dev_i32(cu), cu_seqlens_k=dev_i32(cu), max_seqlen_q=L, max_seqlen_k=L)
    oh, lh = host(o), host(lse)
    g = rng(103, "rows")
    last = L // blk - 1
    for h, m in [(0, last), (1, last), (0, last * 5 // 8), (1, last // 3)]:
        rows = np.sort(g.choice(np.arange(m * blk, m * blk + blk), 6, replace=False))
        wins, cols = oracle.vs_convert_item(L, L, vert[0, h], slash[0, h], m, blk, blk)
        o_ref, lse_ref = oracle.vs_attention_rows(q, k, v, 0, h, rows, wins, cols, cu, cu, blk)
        check_o(oh[rows, h], o_ref, f"vs many columns h={h} m={m}")
        check_lse(lh[h, rows], lse_ref, f"vs many columns lse h={h} m={m}")


@pytest.mark.parametrize("bn", [64, 128])
def test_vs_windows_longer_than_staging(bn):
    """64-row query blocks with more than 256 windows each (slash offsets spread uniformly, so a
    late block's windows cover almost every earlier key): the pair kernel stages 256 windows
    of each block and takes the rest as not shared.  Rows of both blocks of a pair are checked,
    at the end of the sequence (most windows), in the middle and at the start."""
    L, H = 36864, 2
    say(f"vertical-slash with more than 256 windows per block, {bn}-key windows")
    vert, slash = _vs_inputs(105, L, H, 100, 3000)
    q, k, v = (normal_bf16(105, n, (L, H, 128)) for n in ("q", "k", "v"))
    sl = dev_i32([L])
    bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, dev_i32(vert), dev_i32(slash), L, 64, bn)
    assert int(host(bc).max()) > 256
    cu = np.array([0, L], np.int32)
    pat = bsa.VSPattern(bc, bo, cc, ci, 64, bn)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, causal=True, out_dtype=torch.float32,
                         cu_seqlens_q=dev_i32(cu), cu_seqlens_k=dev_i32(cu), max_seqlen_q=L, max_seqlen_k=L)
    oh, lh = host(o), host(lse)
    g = rng(105, "rows")
    last = L // 64 - 1
    for h, m in [(0, last), (1, last - 1), (0, 300), (1, 301), (0, 1)]:
        rows = np.sort(g.choice(np.arange(m * 64, m * 64 + 64), 6, replace=False))
        wins, cols = oracle.vs_convert_item(L, L, vert[0, h], slash[0, h], m, 64, bn)
        o_ref, lse_ref = oracle.vs_attention_rows(q, k, v, 0, h, rows, wins, cols, cu, cu, bn)
        check_o(oh[rows, h], o_ref, f"vs many windows h={h} m={m}")
        check_lse(lh[h, rows], lse_ref, f"vs many windows lse h={h} m={m}")


def test_vs_convert_indices_longer_than_staging():
    """18,000 indices per head, 12,000 of them verticals: the column test walks them in many
    rounds of 64 per query block."""
    L, H, nnz_v, nnz_s = 40000, 1, 12000, 6000
    say("vertical-slash conversion of 18,000 indices per head")
    vert, slash = _vs_inputs(104, L, H, nnz_v, nnz_s)
    sl = dev_i32([L])
    bc, bo, cc, ci = (host(t).astype(np.int64) for t in
                      bsa.vs_convert_indexes(sl, sl, dev_i32(vert), dev_i32(slash), L, 64, 64))
    g = rng(104, "items")
    for m in sorted(set([0, 1, 624] + [int(x) for x in g.integers(0, 625, 12)])):
        wins, cols = oracle.vs_convert_item(L, L, vert[0, 0], slash[0, 0], m, 64, 64)
        assert bc[0, 0, m] == len(wins) and cc[0, 0, m] == len(cols), m
        assert np.array_equal(bo[0, 0, m, :len(wins)], wins), m
        assert np.array_equal(ci[0, 0, m, :len(cols)], cols), m


def test_vs_convert_past_both_staging_limits():
    """The conversion's two global-memory paths: more slash indices per head than the window walk
    stages (16,384) and, on a 280,000-token sequence, late query blocks with more windows than the
    column test stages (4,096).  Sampled items exactly as the oracle converts them."""
    L, H, nnz_v, nnz_s = 280000, 1, 100, 17000
    say("vertical-slash conversion with 17,000 slash indices and more than 4,096 windows per block")
    vert, slash = _vs_inputs(106, L, H, nnz_v, nnz_s)
    sl = dev_i32([L])
    bc, bo, cc, ci = (host(t).astype(np.int64) for t in
                      bsa.vs_convert_indexes(sl, sl, dev_i32(vert), dev_i32(slash), L, 64, 64))
    assert bc.max() > 4096
    last = (L + 63) // 64 - 1
    for m in (0, 1, 2000, last - 1, last):
        wins, cols = oracle.vs_convert_item(L, L, vert[0, 0], slash[0, 0], m, 64, 64)
        assert bc[0, 0, m] == len(wins) and cc[0, 0, m] == len(cols), m
        assert np.array_equal(bo[0, 0, m, :len(wins)], wins), m
        assert np.array_equal(ci[0, 0, m, :len(cols)], cols), m
