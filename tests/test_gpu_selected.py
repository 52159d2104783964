"""GPU parity for selected attention (top-k key blocks per query token): varlen and fixed
length, GQA groups of 1, 2 and 4, causal and not, invalid slots, bf16 output, run-to-run
bit identity (the per-block token lists are filled in a different order every run), and the
full 65536 + 32768-token shape on sampled rows.  Expected values come from the oracle."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import rng
from synth.workloads import selected_prefill
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _run(w, sel=None, causal=True, out_dtype=torch.float32):
    cu = dev_i32(w["cu_seqlens"])
    return bsa.bsa_fwd_selected(dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"]),
                                dev_i32(w["sel"] if sel is None else sel), causal=causal, out_dtype=out_dtype,
                                cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=w["max_seqlen"],
                                max_seqlen_k=w["max_seqlen"])


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2)])
def test_varlen_small(Hq, Hkv):
    w = selected_prefill(seed=71, seqlens=(700, 300, 64), Hq=Hq, Hkv=Hkv, D=128, topk=6)
    say("selected varlen", Hq, Hkv)
    o, lse = _run(w)
    o_ref, lse_ref = oracle.selected(w["q"], w["k"], w["v"], w["sel"], 64, w["cu_seqlens"], w["cu_seqlens"])
    check_o(host(o), o_ref, "selected")
    check_lse(host(lse), lse_ref, "selected lse")


def test_invalid_slots_noncausal_and_bf16():
    """-1 slots, a block past its sequence and blocks after the token (masked when causal,
    attended when not); a token with no slot at all gives (0, -inf)."""
    w = selected_prefill(seed=72, seqlens=(500, 200), Hq=4, Hkv=2, D=128, topk=5)
    sel = w["sel"].copy()
    sel[10, 0] = [0, 3, -1, -1, -1]        # block 3 lies after token 10: causally invisible
    sel[600, 1] = [-1, 1, 4, -1, 2]        # block 4 is past the 200-token second sequence
    sel[650] = -1                          # nothing selected
    say("selected invalid slots")
    o, lse = _run(w, sel)
    ok_sel = sel.copy()
    ok_sel[600, 1] = [-1, 1, -1, -1, 2]    # the oracle rejects blocks past the end: drop it
    o_ref, lse_ref = oracle.selected(w["q"], w["k"], w["v"], ok_sel, 64, w["cu_seqlens"], w["cu_seqlens"])
    check_o(host(o), o_ref, "selected invalid")
    check_lse(host(lse), lse_ref, "selected invalid lse")
    assert np.all(host(o)[650] == 0) and np.isneginf(host(lse)[:, 650]).all()
    say("selected non-causal, bf16 out")
    o, lse = _run(w, ok_sel, causal=False, out_dtype=torch.bfloat16)
    o_ref, lse_ref = oracle.selected(w["q"], w["k"], w["v"], ok_sel, 64, w["cu_seqlens"], w["cu_seqlens"],
                                     causal=False)
    check_o(host(o), o_ref, "selected non-causal", bf16_out=True)
    check_lse(host(lse), lse_ref, "selected non-causal lse")


def test_fixed_length_and_bit_identity():
    w = selected_prefill(seed=73, seqlens=(640, 640), Hq=4, Hkv=2, D=128, topk=7)
    B, S = 2, 640
    q = dev_bf16(w["q"].reshape(B, S, 4, 128))
    k = dev_bf16(w["k"].reshape(B, S, 2, 128))
    v = dev_bf16(w["v"].reshape(B, S, 2, 128))
    sel = dev_i32(w["sel"].reshape(B, S, 2, 7))
    say("selected fixed length")
    o1, l1 = bsa.bsa_fwd_selected(q, k, v, sel, out_dtype=torch.float32)
    o2, l2 = bsa.bsa_fwd_selected(q, k, v, sel, out_dtype=torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "two runs differ"
    o_ref, lse_ref = oracle.selected(w["q"].reshape(B, S, 4, 128), w["k"].reshape(B, S, 2, 128),
                                     w["v"].reshape(B, S, 2, 128), w["sel"].reshape(B, S, 2, 7), 64)
    check_o(host(o1), o_ref, "selected fixed")
    check_lse(host(l1), lse_ref, "selected fixed lse")


@pytest.fixture(scope="module")
def full():
    say("generating selected-attention workload (65536 + 32768 tokens, 4 heads, top-16)")
    w = selected_prefill()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


def test_full_size_sampled(full):
    w = full
    cu = dev_i32(w["cu_seqlens"])
    say("selected full size")
    o, lse = bsa.bsa_fwd_selected(w["dq"], w["dk"], w["dv"], dev_i32(w["sel"]), out_dtype=torch.float32,
                                  cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=65536, max_seqlen_k=65536)
    oh, lh = host(o), host(lse)
    g = rng(6, "rows")
    for b, h in [(0, 0), (0, 3), (1, 1), (1, 2)]:
        L = int(w["seqlens"][b])
        rows = np.sort(np.concatenate([[0, 63, L - 1], g.choice(L, 5, replace=False)]))
        o_ref, lse_ref = oracle.selected_rows(w["q"], w["k"], w["v"], w["sel"], 64, w["cu_seqlens"],
                                              w["cu_seqlens"], b, h, rows)
        a = int(w["cu_seqlens"][b])
        check_o(oh[a + rows, h], o_ref, f"selected full b={b} h={h}")
        check_lse(lh[h, a + rows], lse_ref, f"selected full lse b={b} h={h}")


def test_combine_ignores_o_of_empty_partials():
    """An empty partial (lse -inf) may hold anything in its o, NaN included: the selected path
    writes only the LSE of unused slots and relies on this."""
    g = rng(7, "combine")
    P, B, S, H, D = 3, 1, 16, 2, 128
    o_part = torch.from_numpy(g.standard_normal((P, B, S, H, D)).astype(np.float32)).cuda()
    lse_part = torch.from_numpy(g.standard_normal((P, B, H, S)).astype(np.float32)).cuda()
    lse_part[1] = float("-inf")
    o_part[1] = float("nan")
    o, lse = bsa.bsa_combine(o_part, lse_part, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.combine(host(o_part[[0, 2]]), host(lse_part[[0, 2]]))
    check_o(host(o), o_ref, "combine with an empty NaN partial")
    check_lse(host(lse), lse_ref, "combine with an empty NaN partial lse")
