"""GPU parity for the backward of block-sparse attention (dQ, dK, dV in float32) against the
float64 oracle: dense causal and not (ragged lengths), block lists per query head and per kv
head on 128- and 64-row tiles, and empty lists.  The forward's (O, LSE) come from the GPU path
(float32 O, or bf16 O at full size), as a training step would use them.

Tolerance: per element, twice the worst-case rounding bound of tests/bwd_bound.py: the kernels
round P and dS to bf16 for the MFMA products and sum in float32, so an entry's error is bounded
by the bf16 unit roundoff times the sum of the magnitudes of the products summed into it (plus
the float32 accumulation and the error of the row dot taken from the O the forward handed
over).  Small entries are held to small errors; nothing is measured against the tensor's
largest entry."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import bf16_to_f64, normal_bf16, rng
from synth.workloads import block_sparse_prefill
from tests.bwd_bound import check_within, grad_bounds
from tests.gpu_util import dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _bounds(q, k, v, do, o_used, causal, count=None, index=None, bM=128, bN=128, softcap=0.0):
    """Per-element bounds for the gradients of one fixed-length problem (bf16 bit inputs)."""
    qf, kf, vf, dof = (bf16_to_f64(x) for x in (q, k, v, do))
    Sq, Hq, Sk, Hkv = qf.shape[1], qf.shape[2], kf.shape[1], kf.shape[2]
    cm = oracle.causal_mask(Sq, Sk) if causal else np.ones((Sq, Sk), bool)

    def mask_of(b, h):
        if count is None:
            return cm
        ht = h if count.shape[1] == Hq else h // (Hq // Hkv)
        return cm & oracle.block_mask(count[b, ht], index[b, ht], bM, bN, Sq, Sk)
    return grad_bounds(qf, kf, vf, dof, np.asarray(o_used, np.float64), mask_of, softcap=softcap)


def _data(seed, B, Sq, Sk, Hq, Hkv):
    return (normal_bf16(seed, "q", (B, Sq, Hq, 128)), normal_bf16(seed, "k", (B, Sk, Hkv, 128)),
            normal_bf16(seed, "v", (B, Sk, Hkv, 128)), normal_bf16(seed, "do", (B, Sq, Hq, 128)))


def _grads(q, k, v, do, pattern=None, causal=True, count=None, index=None, bM=128, bN=128, softcap=0.0):
    """GPU gradients, the oracle's, and the per-element bounds (from the GPU forward's O)."""
    dq_, dk_, dv_ = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o, lse = bsa.bsa_fwd(dq_, dk_, dv_, pattern, causal=causal, out_dtype=torch.float32, softcap=softcap)
    g = bsa.bsa_bwd(dq_, dk_, dv_, o, lse, dev_bf16(do), pattern, causal=causal, softcap=softcap)
    ref = oracle.block_sparse_bwd(q, k, v, do, count, index, bM, bN, causal, softcap=softcap)
    bnd = _bounds(q, k, v, do, host(o), causal, count, index, bM, bN, softcap)
    return g, ref, bnd


def _check_all(tag, g, ref, bnd):
    for name, got, r, b in zip(("dq", "dk", "dv"), g, ref, bnd):
        check_within(f"{tag} {name}", host(got), r, b)


@pytest.mark.parametrize("Sq,Sk,causal,B", [(384, 384, True, 2), (300, 456, False, 2), (200, 328, True, 2),
                                            (4096, 4096, True, 1), (2560, 2560, False, 1)])
def test_dense(Sq, Sk, causal, B):
    """The last two cases give key blocks more than 128 slabs of queries: their lists are split
    over several dK/dV workgroups and summed by the reduction (non-causal: every list; causal:
    the early key blocks only)."""
    say("backward dense", Sq, Sk, causal)
    q, k, v, do = _data(91, B, Sq, Sk, 4, 2)
    _check_all(f"dense {Sq}x{Sk} causal={causal}", *_grads(q, k, v, do, None, causal))


def _lists(seed, B, H, nqb, nkb, cap):
    g = rng(seed, "bwd-lists")
    count = np.zeros((B, H, nqb), np.int32)
    index = np.zeros((B, H, nqb, cap), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                reach = min(i, nkb - 1)
                pool = np.arange(reach)
                n = int(g.integers(0, min(cap - 1, pool.size) + 1)) if pool.size else 0
                sel = np.concatenate([[reach], g.choice(pool, n, replace=False)]) if n else np.array([reach])
                sel = g.permutation(sel)
                count[b, h, i] = sel.size
                index[b, h, i, :sel.size] = sel
    return count, index


@pytest.mark.parametrize("bM,bN,Ht", [(128, 128, "q"), (128, 128, "kv"), (64, 64, "q"), (64, 128, "kv")])
def test_block_lists(bM, bN, Ht):
    B, S, Hq, Hkv = 2, 512, 4, 2
    say("backward block lists", bM, bN, Ht)
    q, k, v, do = _data(92, B, S, S, Hq, Hkv)
    H = Hq if Ht == "q" else Hkv
    nqb, nkb = S // bM, S // bN
    # query block i of bM rows reaches key block (i*bM + bM - 1) // bN
    count, index = _lists(92, B, H, nqb, nkb, 4)
    for i in range(nqb):
        index[:, :, i] = np.minimum(index[:, :, i], ((i + 1) * bM - 1) // bN)
        for b in range(B):
            for h in range(H):
                row = index[b, h, i, :count[b, h, i]]
                u = np.unique(row)
                count[b, h, i] = u.size
                index[b, h, i, :u.size] = u
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, bN)
    _check_all(f"lists {bM}x{bN} {Ht}", *_grads(q, k, v, do, pat, True, count, index, bM, bN))


@pytest.mark.parametrize("kind,causal", [("dense", True), ("dense", False), ("block", True)])
def test_softcap(kind, causal):
    """Soft-capped scores (cap 1.5, so that the scaled scores, of size about 1, are far into the
    nonlinear part of c tanh(x / c)): the gradient carries the factor 1 - tanh^2."""
    B, Sq, Sk, Hq, Hkv, cap = 2, 384, 456 if not causal else 384, 4, 2, 1.5
    say("backward softcap", kind, causal)
    q, k, v, do = _data(96, B, Sq, Sk, Hq, Hkv)
    count = index = pat = None
    if kind == "block":
        count, index = _lists(96, B, Hq, Sq // 128, Sk // 128, 3)
        pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), 128, 128)
    g, ref, bnd = _grads(q, k, v, do, pat, causal, count, index, softcap=cap)
    _check_all(f"softcap {kind} causal={causal}", g, ref, bnd)
    rq = ref[0]
    # the cap matters: the uncapped gradient is far from the capped one
    r0 = oracle.block_sparse_bwd(q, k, v, do, count, index, 128, 128, causal)[0]
    assert np.abs(r0 - rq).max() > 0.1 * max(1.0, np.abs(rq).max())


def test_empty_lists_give_zero_rows():
    B, S, Hq, Hkv = 1, 256, 2, 2
    say("backward empty lists")
    q, k, v, do = _data(93, B, S, S, Hq, Hkv)
    count = np.full((B, Hq, 2), 2, np.int32)
    index = np.broadcast_to(np.array([0, 1], np.int32), (B, Hq, 2, 2)).copy()
    count[0, 1, 1] = 0
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), 128, 128)
    g, ref, bnd = _grads(q, k, v, do, pat, True, count, index)
    assert np.all(host(g[0])[0, 128:, 1] == 0)
    _check_all("empty lists", g, ref, bnd)


@pytest.mark.parametrize("Ht", ["q", "kv"])
def test_long_lists_split_and_repeat_bit_for_bit(Ht):
    """Key block 0 is named by every query block, so its dK/dV list (G heads x 32 query blocks x
    4 slabs) is cut into several chunks and reduced; two runs give the same bits (the lists are
    built in a fixed order)."""
    B, S, Hq, Hkv, bM = 1, 4096, 8, 2, 128
    say("backward long lists", Ht)
    q, k, v, do = _data(94, B, S, S, Hq, Hkv)
    H = Hq if Ht == "q" else Hkv
    nqb = S // bM
    g = rng(94, "long-lists")
    cap = 6
    count = np.zeros((B, H, nqb), np.int32)
    index = np.zeros((B, H, nqb, cap), np.int32)
    for h in range(H):
        for i in range(nqb):
            extra = g.choice(np.arange(1, i), min(cap - 2, max(i - 1, 0)), replace=False) if i > 1 else []
            sel = np.unique(np.concatenate([[0, i], extra]).astype(np.int32))
            count[0, h, i] = sel.size
            index[0, h, i, :sel.size] = g.permutation(sel)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, 128)
    _check_all(f"long lists {Ht}", *_grads(q, k, v, do, pat, True, count, index))
    dq_, dk_, dv_ = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o, lse = bsa.bsa_fwd(dq_, dk_, dv_, pat, causal=True, out_dtype=torch.float32)
    dO = dev_bf16(do)
    first = bsa.bsa_bwd(dq_, dk_, dv_, o, lse, dO, pat, causal=True)
    for _ in range(2):
        again = bsa.bsa_bwd(dq_, dk_, dv_, o, lse, dO, pat, causal=True)
        for a_, b_ in zip(first, again):
            assert torch.equal(a_, b_), "backward runs differ"


@pytest.mark.parametrize("kind,softcap", [("dense", 0.0), ("block", 0.0), ("block", 2.0)])
def test_varlen(kind, softcap):
    """Packed variable-length sequences (differing query and key lengths, partial last blocks),
    with and without softcap: each sequence's gradients are those of its own fixed-length
    problem."""
    q_lens, k_lens, Hq, Hkv, bM, bN = (300, 129, 512), (420, 129, 512), 4, 2, 128, 64
    say("backward varlen", kind, softcap)
    cq = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    q = normal_bf16(95, "q", (int(cq[-1]), Hq, 128))
    k = normal_bf16(95, "k", (int(ck[-1]), Hkv, 128))
    v = normal_bf16(95, "v", (int(ck[-1]), Hkv, 128))
    do = normal_bf16(95, "do", (int(cq[-1]), Hq, 128))
    B, nqb = len(q_lens), -(-max(q_lens) // bM)
    count = index = pat = None
    if kind == "block":
        g = rng(95, "varlen-bwd-lists")
        cap = 5
        count = np.zeros((B, Hq, nqb), np.int32)
        index = np.full((B, Hq, nqb, cap), 99, np.int32)  # junk past the counts and the sequences
        for b in range(B):
            nkb = -(-k_lens[b] // bN)
            for h in range(Hq):
                for i in range(-(-q_lens[b] // bM)):
                    n = int(g.integers(1, min(cap, nkb) + 1))
                    count[b, h, i] = n
                    index[b, h, i, :n] = g.choice(nkb, n, replace=False)
        pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, bN)
    varlen = dict(cu_seqlens_q=dev_i32(cq), cu_seqlens_k=dev_i32(ck), max_seqlen_q=max(q_lens),
                  max_seqlen_k=max(k_lens))
    dq_, dk_, dv_ = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for causal in (True, False):
        o, lse = bsa.bsa_fwd(dq_, dk_, dv_, pat, causal=causal, out_dtype=torch.float32, softcap=softcap, **varlen)
        gq, gk, gv = bsa.bsa_bwd(dq_, dk_, dv_, o, lse, dev_bf16(do), pat, causal=causal, softcap=softcap, **varlen)
        gq, gk, gv, oh = host(gq), host(gk), host(gv), host(o)
        for b in range(B):
            qs, ks = slice(int(cq[b]), int(cq[b + 1])), slice(int(ck[b]), int(ck[b + 1]))
            nq = -(-q_lens[b] // bM)
            cnt = None if count is None else count[b:b + 1, :, :nq]
            idx = None if index is None else index[b:b + 1, :, :nq]
            rq, rk, rv = oracle.block_sparse_bwd(q[qs][None], k[ks][None], v[ks][None], do[qs][None], cnt, idx,
                                                 bM, bN, causal, softcap=softcap)
            bq, bk, bv = _bounds(q[qs][None], k[ks][None], v[ks][None], do[qs][None], oh[qs][None], causal, cnt, idx,
                                 bM, bN, softcap)
            for name, got, ref, bd in (("dq", gq[qs], rq[0], bq[0]), ("dk", gk[ks], rk[0], bk[0]),
                                       ("dv", gv[ks], rv[0], bv[0])):
                check_within(f"varlen {kind} cap={softcap} causal={causal} seq {b} {name}", got, ref, bd)


@pytest.fixture(scope="module")
def bwd_full():
    say("generating block-sparse causal prefill workload and upstream gradient (S=32768, Hq=32, Hkv=8)")
    w = block_sparse_prefill()
    w["do"] = normal_bf16(1007, "do", w["q"].shape)
    return w


def _packed(w, h, i, oh):
    """Query block i of query head h against the key blocks its list names, packed in ascending
    order: every listed block but the diagonal one lies wholly before the block's rows, and the
    diagonal block comes last, so bottom-right causal masking of the packed keys is the original
    mask.  Returns the sorted block ids, the oracle's (dq, dk, dv) of that small problem and
    their bounds (oh: the GPU forward's O, which the kernels used)."""
    hk = h // (w["Hq"] // w["Hkv"])
    ents = np.sort(w["index"][0, h, i, :w["count"][0, h, i]])
    rows = slice(i * 128, (i + 1) * 128)
    keys = np.concatenate([np.arange(j * 128, (j + 1) * 128) for j in ents])
    args = (w["q"][:, rows, h:h + 1], w["k"][:, keys, hk:hk + 1], w["v"][:, keys, hk:hk + 1], w["do"][:, rows, h:h + 1])
    return ents, oracle.block_sparse_bwd(*args, causal=True), _bounds(*args, oh[:, rows, h:h + 1], True)


def test_full_size_sampled(bwd_full):
    """The block-sparse causal prefill at full size (S=32768, Hq=32, Hkv=8, 128x128 tiles, bf16 O
    from the forward), launched as the benchmark launches it.  Sampled: dQ of 16 query blocks
    (first and last included, spread over the heads); dK and dV of the last key block (seen by
    the diagonal tiles only), of key blocks 128 and 200, and of key block 1, which several hundred
    (head, query block) lists name, so its sums are split over many chunks and go through the
    reduction.  Each expected block sums the oracle's gradients of the small packed problems of
    every (head, query block) that names it."""
    w = bwd_full
    say("backward full size")
    q, k, v, do = (dev_bf16(w[n]) for n in ("q", "k", "v", "do"))
    pat = bsa.BlockPattern(dev_i32(w["count"]), dev_i32(w["index"]), 128, 128)
    o, lse = bsa.bsa_fwd(q, k, v, pat, causal=True, out_dtype=torch.bfloat16)
    ws = torch.empty(bsa.bsa_bwd_workspace_size(q, k, pat, causal=True), dtype=torch.uint8, device=q.device)
    gq, gk, gv = bsa.bsa_bwd(q, k, v, o, lse, do, pat, causal=True, workspace=ws)
    oh = host(o)
    gq, gk, gv = host(gq), host(gk), host(gv)
    for h, i in [(0, 255), (31, 0), (12, 200), (1, 1), (2, 17), (5, 254), (7, 99), (9, 128), (14, 31), (16, 64),
                 (19, 177), (21, 240), (24, 3), (26, 150), (28, 211), (30, 90)]:
        _, (rq, _, _), (bq, _, _) = _packed(w, h, i, oh)
        check_within(f"full dq h={h} i={i}", gq[0, i * 128:(i + 1) * 128, h], rq[0, :, 0], bq[0, :, 0])
    G = w["Hq"] // w["Hkv"]
    nqb = w["count"].shape[2]
    for hk, j in [(3, nqb - 1), (0, 128), (7, 200), (5, 1)]:
        rk = np.zeros((128, 128))
        rv = np.zeros((128, 128))
        bk = np.zeros((128, 128))
        bv = np.zeros((128, 128))
        named = 0
        for h in range(hk * G, (hk + 1) * G):
            for i in range(j, nqb):
                if j not in w["index"][0, h, i, :w["count"][0, h, i]]:
                    continue
                ents, (_, sk, sv), (_, ek, ev) = _packed(w, h, i, oh)
                p = int(np.searchsorted(ents, j)) * 128
                rk += sk[0, p:p + 128, 0]
                rv += sv[0, p:p + 128, 0]
                bk += ek[0, p:p + 128, 0]          # the sum of the lists' bounds bounds the sum
                bv += ev[0, p:p + 128, 0]
                named += 1
        say(f"key block {j} of kv head {hk}: named by {named} lists")
        check_within(f"full dk hk={hk} j={j}", gk[0, j * 128:(j + 1) * 128, hk], rk, bk)
        check_within(f"full dv hk={hk} j={j}", gv[0, j * 128:(j + 1) * 128, hk], rv, bv)
