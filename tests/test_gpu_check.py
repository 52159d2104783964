"""GPU tests of the pattern check (bsa_check_pattern) and of the debug mode that runs it in
front of the attention entry points (BSA_DEBUG_CHECKS): valid block lists and valid output of
the vertical-slash conversion pass; planted violations are each found, with the first one
named; varlen lists past a sequence's own query blocks are ignored; with the variable set, a
bad pattern is refused before launch and a good one gives the same bits as without it."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
from synth import normal_bf16, rng
from synth.workloads import vs_varlen_prefill
from tests.gpu_util import dev_bf16, dev_i32, say

pytestmark = [pytest.mark.gpu]

NONE = 2**31 - 1
B, Hq, Hkv, S, D, BM, BN, CAP = 2, 4, 2, 1024, 128, 128, 64, 6
NQB, NKB = S // BM, S // BN


def _flat(b, h, m, Ht=Hq, nqb=NQB):
    return (b * Ht + h) * nqb + m


def _block_lists(seed):
    """Valid lists: at most CAP distinct in-range ids; unused slots hold junk."""
    g = rng(seed, "check lists")
    count = g.integers(0, CAP + 1, size=(B, Hq, NQB)).astype(np.int32)
    index = np.full((B, Hq, NQB, CAP), 12345, np.int32)
    for b in range(B):
        for h in range(Hq):
            for m in range(NQB):
                n = count[b, h, m]
                index[b, h, m, :n] = g.choice(NKB, n, replace=False)
    return count, index


def _qkv(seed, Sq=S):
    q = dev_bf16(normal_bf16(seed, "q", (B, Sq, Hq, D)))
    k = dev_bf16(normal_bf16(seed, "k", (B, S, Hkv, D)))
    v = dev_bf16(normal_bf16(seed, "v", (B, S, Hkv, D)))
    return q, k, v


def _pattern(count, index):
    return bsa.BlockPattern(dev_i32(count), dev_i32(index), BM, BN)


def _check(q, k, pat, **kw):
    r = bsa.bsa_check_pattern(q, k, pat, **kw)
    torch.cuda.synchronize()
    r = r.cpu().numpy()
    return int(r[0]), int(r[1])


def test_block_lists():
    q, k, _ = _qkv(81)
    count, index = _block_lists(81)
    say("check block lists: valid")
    assert _check(q, k, _pattern(count, index)) == (0, NONE)
    planted = []
    c, x = count.copy(), index.copy()

    def plant(b, h, m):
        planted.append(_flat(b, h, m))

    c[0, 1, 2] = 3; x[0, 1, 2, :3] = [4, 9, 4]; plant(0, 1, 2)            # repeated id
    c[1, 3, 0] = 2; x[1, 3, 0, :2] = [1, NKB]; plant(1, 3, 0)             # id past the keys
    c[1, 0, 3] = CAP + 1; plant(1, 0, 3)                                  # count above cap
    c[0, 2, 5] = 1; x[0, 2, 5, 0] = -1; plant(0, 2, 5)                    # negative id
    c[1, 2, 7] = -1; plant(1, 2, 7)                                       # negative count
    c[0, 0, 6] = 1; x[0, 0, 6, 0] = 0; x[0, 0, 6, 1:] = 0                 # junk past count: fine
    say("check block lists: planted", len(planted))
    assert _check(q, k, _pattern(c, x)) == (len(planted), min(planted))
    # lists per kv head (Ht = Hkv) with strides of that shape
    ck, xk = count[:, :Hkv].copy(), index[:, :Hkv].copy()
    assert _check(q, k, _pattern(ck, xk)) == (0, NONE)
    ck[1, 1, 4] = 2; xk[1, 1, 4, :2] = [3, 3]
    assert _check(q, k, _pattern(ck, xk)) == (1, _flat(1, 1, 4, Ht=Hkv))


def test_broadcast_table_and_decode_shape():
    q, k, _ = _qkv(82, Sq=1)
    say("check 1-D table (decode)")
    good = bsa.BlockPattern.table(dev_i32(np.arange(0, NKB, 3)), BN)
    assert _check(q, k, good) == (0, NONE)
    bad = bsa.BlockPattern.table(dev_i32([0, 5, 5]), BN)
    # one table shared by every list: every (b, h) list is flagged, the first is list 0
    assert _check(q, k, bad) == (B * Hq, 0)


def _vs(seed=83, seqlens=(300, 170), ctx=320):
    w = vs_varlen_prefill(seed=seed, seqlens=seqlens, H=Hq, D=D, nnz_v=20, nnz_s=12, block=64, context_size=ctx)
    sl = dev_i32(w["seqlens"])
    conv = bsa.vs_convert_indexes(sl, sl, dev_i32(w["vertical"]), dev_i32(w["slash"]), ctx, 64, 64)
    cu = dev_i32(w["cu_seqlens"])
    varlen = dict(cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=int(max(seqlens)), max_seqlen_k=int(max(seqlens)))
    torch.cuda.synchronize()
    return w, [t.cpu().numpy() for t in conv], varlen


def _vs_pattern(bc, bo, cc, ci):
    return bsa.VSPattern(dev_i32(bc), dev_i32(bo), dev_i32(cc), dev_i32(ci), 64, 64)


def test_vertical_slash():
    w, (bc, bo, cc, ci), varlen = _vs()
    q, k = dev_bf16(w["q"]), dev_bf16(w["k"])
    nqb = -(-int(max(w["seqlens"])) // 64)
    kw = dict(causal=True, **varlen)
    say("check vertical-slash: converter output")
    assert _check(q, k, _vs_pattern(bc, bo, cc, ci), **kw) == (0, NONE)
    # rows past the 170-token sequence's own query blocks are never read: junk there is fine
    bc2 = bc.copy()
    bc2[1, :, 3:] = 99
    assert _check(q, k, _vs_pattern(bc2, bo, cc, ci), **kw) == (0, NONE)

    bc2, bo2, cc2, ci2 = bc.copy(), bo.copy(), cc.copy(), ci.copy()
    cand = [(b, h, m) for b in range(2) for h in range(Hq) for m in range(3)]
    planted = []

    def pick(ok):
        t = next(t for t in cand if ok(t) and t not in planted)
        planted.append(t)
        return t

    t = pick(lambda t: cc[t] >= 2); ci2[t][:2] = ci2[t][1::-1]                      # columns out of order
    t = pick(lambda t: bc[t] >= 1); bc2[t] = 2; bo2[t][1] = bo2[t][0] + 32          # overlapping windows
    t = pick(lambda t: bc[t] >= 1); cc2[t] = 1; ci2[t][0] = bo2[t][0] + 5           # column inside a window
    t = pick(lambda t: True); cc2[t] = ci.shape[-1] + 1                            # column count above cap
    say("check vertical-slash: planted", len(planted))
    got = _check(q, k, _vs_pattern(bc2, bo2, cc2, ci2), **kw)
    assert got == (4, min(_flat(b, h, m, nqb=nqb) for b, h, m in planted))


def test_debug_mode_refuses_bad_patterns(monkeypatch):
    q, k, v = _qkv(84)
    count, index = _block_lists(84)
    good = _pattern(count, index)
    c, x = count.copy(), index.copy()
    c[1, 2, 3] = 2; x[1, 2, 3, :2] = [7, 7]
    bad = _pattern(c, x)
    say("debug mode off: bad pattern not inspected")
    o_ref, lse_ref = bsa.bsa_fwd(q, k, v, good, causal=True, out_dtype=torch.float32)
    monkeypatch.setenv("BSA_DEBUG_CHECKS", "1")
    say("debug mode: bsa_fwd")
    o, lse = bsa.bsa_fwd(q, k, v, good, causal=True, out_dtype=torch.float32)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    with pytest.raises(bsa.BSAError) as e:
        bsa.bsa_fwd(q, k, v, bad, causal=True)
    assert e.value.status == 1
    say("debug mode: bsa_fwd_partials")
    with pytest.raises(bsa.BSAError):
        bsa.bsa_fwd_partials(q, k, v, bad, 2, causal=True)
    say("debug mode: bsa_bwd")
    dout = dev_bf16(normal_bf16(84, "dout", (B, S, Hq, D)))
    with pytest.raises(bsa.BSAError):
        bsa.bsa_bwd(q, k, v, o_ref, lse_ref, dout, bad, causal=True)
    say("debug mode: speculative decode")
    qd = q[:, -1:].contiguous()
    miss_ok = bsa.BlockPattern(dev_i32(count[:, :, :1]), dev_i32(index[:, :, :1]), BM, BN)
    miss_bad = bsa.BlockPattern(dev_i32(c[:, :, 3:4]), dev_i32(x[:, :, 3:4]), BM, BN)
    o1, l1 = bsa.speculative_sparse(qd, k[:, :256], v[:, :256], k, v, miss_ok, out_dtype=torch.float32)
    with pytest.raises(bsa.BSAError):
        bsa.speculative_sparse(qd, k[:, :256], v[:, :256], k, v, miss_bad)
    monkeypatch.setenv("BSA_DEBUG_CHECKS", "0")
    o2, l2 = bsa.speculative_sparse(qd, k[:, :256], v[:, :256], k, v, miss_ok, out_dtype=torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
