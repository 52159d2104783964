"""GPU parity for the prefill path: block-sparse causal prefill (small, ragged and full size),
dense prefill, per-key/value-head lists, 64-row tiles, and partials.  Expected values come from
the float64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import normal_bf16, rng
from synth.workloads import block_sparse_prefill
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _lists(seed, B, H, reach, cap):
    """Random block lists per (b, h, query block i): the last causally reachable block
    reach[i], block 0 and random blocks in between; counts vary; order is shuffled (order
    must not matter)."""
    g = rng(seed, "lists")
    nqb = len(reach)
    count = np.zeros((B, H, nqb), np.int32)
    index = np.zeros((B, H, nqb, cap), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                sel = {int(reach[i]), 0}
                pool = np.arange(1, reach[i])
                k = int(g.integers(0, min(cap - len(sel), pool.size) + 1)) if pool.size else 0
                if k:
                    sel.update(g.choice(pool, size=k, replace=False).tolist())
                sel = g.permutation(sorted(sel))
                count[b, h, i] = sel.size
                index[b, h, i, :sel.size] = sel
    return count, index


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,Ht,bM,bN", [
    (1024, 1024, 8, 2, "q", 128, 128),     # several query tiles, GQA, lists per query head
    (1000, 1024, 4, 2, "kv", 128, 128),    # ragged query tail, bottom-right causal offset 24
    (512, 512, 4, 4, "q", 64, 64),         # 64-row tiles (two waves), 64-key blocks
    (384, 512, 4, 2, "q", 128, 64),        # 128-row tiles over 64-key blocks
    (448, 512, 4, 2, "kv", 64, 128),       # 64-row tiles over 128-key blocks (four 32-key chunks each)
])
def test_block_sparse_causal_small(Sq, Sk, Hq, Hkv, Ht, bM, bN):
    B, D = 2, 128
    say("block-sparse prefill", Sq, Sk, Hq, Hkv, Ht, bM, bN)
    q = normal_bf16(11, "q", (B, Sq, Hq, D))
    k = normal_bf16(11, "k", (B, Sk, Hkv, D))
    v = normal_bf16(11, "v", (B, Sk, Hkv, D))
    H = Hq if Ht == "q" else Hkv
    nqb = -(-Sq // bM)
    reach = [(min(Sq, (i + 1) * bM) - 1 + Sk - Sq) // bN for i in range(nqb)]
    count, index = _lists(11, B, H, reach, 6)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, bN)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, causal=True, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, count, index, bM, bN, causal=True)
    check_o(host(o), o_ref, "block-sparse")
    check_lse(host(lse), lse_ref, "block-sparse lse")


@pytest.mark.parametrize("Sq,Sk,causal", [(640, 640, True), (300, 700, False), (257, 257, True)])
def test_dense_prefill(Sq, Sk, causal):
    B, Hq, Hkv, D = 1, 8, 2, 128
    say("dense prefill", Sq, Sk, causal)
    q = normal_bf16(12, "q", (B, Sq, Hq, D))
    k = normal_bf16(12, "k", (B, Sk, Hkv, D))
    v = normal_bf16(12, "v", (B, Sk, Hkv, D))
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), None, causal=causal, out_dtype=torch.bfloat16)
    o_ref, lse_ref = oracle.dense(q, k, v, causal=causal)
    check_o(host(o), o_ref, "dense prefill (bf16 out)", bf16_out=True)
    check_lse(host(lse), lse_ref, "dense prefill lse")


@pytest.mark.parametrize("E,bM,bN", [(1, 128, 128), (3, 128, 128), (2, 64, 128)])
def test_prefill_partials_recombine(E, bM, bN):
    B, S, Hq, Hkv, D = 1, 512, 4, 2, 128
    say("prefill partials E =", E, bM, bN)
    q = normal_bf16(13, "q", (B, S, Hq, D))
    k = normal_bf16(13, "k", (B, S, Hkv, D))
    v = normal_bf16(13, "v", (B, S, Hkv, D))
    nqb, nkb = S // bM, S // bN
    count = np.zeros((B, Hq, nqb), np.int32)
    index = np.zeros((B, Hq, nqb, nkb), np.int32)
    for i in range(nqb):
        reach = ((i + 1) * bM - 1) // bN  # every block up to the diagonal, diagonal first
        count[0, :, i] = reach + 1
        index[0, :, i, :reach + 1] = np.arange(reach + 1)[::-1]
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, bN)
    op, lp = bsa.bsa_fwd_partials(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, E, causal=True)
    if E == 1:
        op_ref, lp_ref = oracle.block_sparse_partials(q, k, v, count, index, bM, bN, causal=True)
        check_o(host(op), op_ref, "partials")
        check_lse(host(lp), lp_ref, "partials lse")
    o, lse = bsa.bsa_combine(op, lp, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, count, index, bM, bN, causal=True)
    check_o(host(o), o_ref, "recombined")
    check_lse(host(lse), lse_ref, "recombined lse")


def test_empty_lists_prefill():
    B, S, H, D = 1, 256, 2, 128
    say("empty lists prefill")
    q = normal_bf16(14, "q", (B, S, H, D))
    k = normal_bf16(14, "k", (B, S, H, D))
    v = normal_bf16(14, "v", (B, S, H, D))
    count = np.array([[[0, 1], [2, 0]]], np.int32)
    index = np.array([[[[0, 0], [0, 0]], [[1, 0], [0, 0]]]], np.int32)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), 128, 128)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, causal=False, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, count, index, 128, 128)
    check_o(host(o), o_ref, "empty lists")
    check_lse(host(lse), lse_ref, "empty lists lse")


@pytest.fixture(scope="module")
def cfg3():
    say("generating block-sparse causal prefill workload (S=32768, Hq=32, Hkv=8)")
    w = block_sparse_prefill()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


def test_block_sparse_full_size(cfg3):
    """Every row of 16 query blocks across the heads, the first and last blocks included."""
    w = cfg3
    say("block-sparse prefill full size")
    pat = bsa.BlockPattern(dev_i32(w["count"]), dev_i32(w["index"]), 128, 128)
    o, lse = bsa.bsa_fwd(w["dq"], w["dk"], w["dv"], pat, causal=True, out_dtype=torch.float32)
    oh, lh = host(o), host(lse)
    scale = 1.0 / np.sqrt(128)
    blocks = [(0, 255), (31, 255), (31, 0), (7, 1), (19, 33), (12, 200), (25, 128), (3, 34), (4, 35),
              (5, 254), (8, 100), (13, 64), (16, 17), (22, 240), (27, 2), (30, 190)]
    for h, i in blocks:
        rows = np.arange(i * 128, (i + 1) * 128)
        ents = w["index"][0, h, i, :w["count"][0, h, i]]
        ks = np.concatenate([np.arange(j * 128, (j + 1) * 128) for j in ents])
        o_ref, lse_ref = oracle.attend_rows(w["q"][0, rows, h], w["k"][0, :, h // 4], w["v"][0, :, h // 4],
                                            [ks[ks <= r] for r in rows], scale)
        check_o(oh[0, rows, h], o_ref, f"full h={h} i={i}")
        check_lse(lh[0, h, rows], lse_ref, f"full lse h={h} i={i}")
