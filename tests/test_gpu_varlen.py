"""GPU parity for packed variable-length prefill (cu_seqlens) with dense and block-list
patterns, causal and not, query and key lengths that differ per sequence and are not
multiples of the tile sizes.  Variable-length attention is the fixed-length attention of each
sequence on its own, so the expected values are the oracle's, one sequence at a time."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import normal_bf16, rng
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

D, Hq, Hkv = 128, 4, 2


def _inputs(seed, q_lens, k_lens):
    cq = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
    q = normal_bf16(seed, "q", (int(cq[-1]), Hq, D))
    k = normal_bf16(seed, "k", (int(ck[-1]), Hkv, D))
    v = normal_bf16(seed, "v", (int(ck[-1]), Hkv, D))
    return q, k, v, cq, ck


def _run(q, k, v, cq, ck, q_lens, k_lens, pattern, causal):
    return bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pattern, causal=causal, out_dtype=torch.float32,
                       cu_seqlens_q=dev_i32(cq), cu_seqlens_k=dev_i32(ck), max_seqlen_q=int(max(q_lens)),
                       max_seqlen_k=int(max(k_lens)))


def _check(o, lse, refs, cq, what):
    oh, lh = host(o), host(lse)
    for b, (o_ref, lse_ref) in enumerate(refs):
        a, e = int(cq[b]), int(cq[b + 1])
        check_o(oh[a:e], o_ref[0], f"{what} seq {b}")
        check_lse(lh[:, a:e], lse_ref[0], f"{what} lse seq {b}")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_dense(causal):
    q_lens, k_lens = (300, 129, 512), (300, 200, 512)
    say("varlen dense", causal)
    q, k, v, cq, ck = _inputs(111, q_lens, k_lens)
    o, lse = _run(q, k, v, cq, ck, q_lens, k_lens, None, causal)
    refs = [oracle.dense(q[cq[b]:cq[b + 1]][None], k[ck[b]:ck[b + 1]][None], v[ck[b]:ck[b + 1]][None], causal)
            for b in range(len(q_lens))]
    _check(o, lse, refs, cq, f"varlen dense causal={causal}")


@pytest.mark.parametrize("Ht,bM,bN", [("q", 128, 128), ("kv", 128, 64), ("q", 64, 64)])
def test_varlen_block_lists(Ht, bM, bN):
    q_lens, k_lens = (300, 129, 512), (420, 129, 512)
    say("varlen block lists", Ht, bM, bN)
    q, k, v, cq, ck = _inputs(112, q_lens, k_lens)
    H = Hq if Ht == "q" else Hkv
    B, nqb, cap = len(q_lens), -(-max(q_lens) // bM), 5
    g = rng(112, f"varlen lists {Ht}")
    count = np.zeros((B, H, nqb), np.int32)
    index = np.full((B, H, nqb, cap), 77, np.int32)
    for b in range(B):
        nkb = -(-k_lens[b] // bN)  # blocks of this sequence (the last one partial)
        for h in range(H):
            for i in range(nqb):
                n = int(g.integers(0, min(cap, nkb) + 1))
                count[b, h, i] = n
                index[b, h, i, :n] = g.choice(nkb, n, replace=False)
    pat = bsa.BlockPattern(dev_i32(count), dev_i32(index), bM, bN)
    for causal in (True, False):
        o, lse = _run(q, k, v, cq, ck, q_lens, k_lens, pat, causal)
        refs = []
        for b in range(B):
            nq = -(-q_lens[b] // bM)
            refs.append(oracle.block_sparse(q[cq[b]:cq[b + 1]][None], k[ck[b]:ck[b + 1]][None],
                                            v[ck[b]:ck[b + 1]][None], count[b:b + 1, :, :nq],
                                            index[b:b + 1, :, :nq], bM, bN, causal))
        _check(o, lse, refs, cq, f"varlen block {Ht} {bM}x{bN} causal={causal}")
