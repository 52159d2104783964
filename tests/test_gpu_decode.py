"""GPU parity for the decode path (few query rows per key/value head): tiny sparse decode,
per-entry partials, the combine, speculative + sparse decode at small and full size, and edge
cases.  Every expected value comes from the float64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth import normal_bf16, rng
from synth.workloads import spec_sparse_decode, tiny_decode
from tests.gpu_util import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _pattern_kv(lists, block_N, Ht_lists):
    """BlockPattern with one list per (b, h) for a single query block."""
    B, H, n = lists.shape
    count = np.full((B, H, 1), n, np.int32)
    return bsa.BlockPattern(dev_i32(count), dev_i32(lists.reshape(B, H, 1, n)), 128, block_N), count, \
        lists.reshape(B, H, 1, n)


@pytest.fixture(scope="module")
def tiny():
    w = tiny_decode()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


@pytest.mark.parametrize("which", ["set_a", "set_b", "full"])
def test_tiny_decode_sets(tiny, which):
    say("tiny decode", which)
    pat, cnt, idx = _pattern_kv(tiny[which], 64, tiny["Hkv"])
    o, lse = bsa.bsa_fwd(tiny["dq"], tiny["dk"], tiny["dv"], pat, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(tiny["q"], tiny["k"], tiny["v"], cnt, idx, 1, 64)
    check_o(host(o), o_ref, which)
    check_lse(host(lse), lse_ref, which)


def test_tiny_decode_combine_identity(tiny):
    say("tiny decode combine(A, B) vs full and dense")
    pa, ca, ia = _pattern_kv(tiny["set_a"], 64, 4)
    pb, cb, ib = _pattern_kv(tiny["set_b"], 64, 4)
    o_part = torch.empty((2, 1, 1, 4, 64), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((2, 1, 4, 1), dtype=torch.float32, device="cuda")
    bsa.bsa_fwd(tiny["dq"], tiny["dk"], tiny["dv"], pa, out=o_part[0], lse=lse_part[0])
    bsa.bsa_fwd(tiny["dq"], tiny["dk"], tiny["dv"], pb, out=o_part[1], lse=lse_part[1])
    o, lse = bsa.bsa_combine(o_part, lse_part, out_dtype=torch.float32)
    od, lsed = bsa.bsa_fwd(tiny["dq"], tiny["dk"], tiny["dv"], None, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.dense(tiny["q"], tiny["k"], tiny["v"])
    for name, oo, ll in (("combine", o, lse), ("dense", od, lsed)):
        check_o(host(oo), o_ref, name)
        check_lse(host(ll), lse_ref, name)


def test_tiny_decode_partials(tiny):
    say("tiny decode per-entry partials")
    pa, ca, ia = _pattern_kv(tiny["set_a"], 64, 4)
    op, lp = bsa.bsa_fwd_partials(tiny["dq"], tiny["dk"], tiny["dv"], pa)
    op_ref, lp_ref = oracle.block_sparse_partials(tiny["q"], tiny["k"], tiny["v"], ca, ia, 1, 64)
    check_o(host(op), op_ref, "partials")
    check_lse(host(lp), lp_ref, "partials lse")
    o, lse = bsa.bsa_combine(op, lp, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(tiny["q"], tiny["k"], tiny["v"], ca, ia, 1, 64)
    check_o(host(o), o_ref, "combined partials")
    check_lse(host(lse), lse_ref, "combined partials lse")


def _small_spec(seed=77, B=2, Hq=8, Hkv=2, D=128, Sk=4096, bs=64):
    return spec_sparse_decode(seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, Sk=Sk, bs=bs, spec_tokens=512)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_speculative_small(out_dtype):
    w = _small_spec()
    say("speculative+sparse small", out_dtype)
    q, k, v = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    s0 = w["spec_start"]
    missed, cnt, idx = _pattern_kv(w["missed"], 64, w["Hkv"])
    o, lse = bsa.speculative_sparse(q, k[:, s0:], v[:, s0:], k, v, missed, causal_spec=True, out_dtype=out_dtype)
    o_ref, lse_ref = oracle.speculative_sparse(w["q"], w["k"][:, s0:], w["v"][:, s0:], w["k"], w["v"], cnt, idx, 64,
                                               causal_spec=True)
    check_o(host(o), o_ref, "spec", bf16_out=out_dtype == torch.bfloat16)
    check_lse(host(lse), lse_ref, "spec lse")


def test_list_per_query_head_and_block128():
    """Lists per query head (no GQA sharing: one head per workgroup) with 128-key blocks."""
    B, Hq, Hkv, D, Sk = 2, 8, 2, 128, 2048
    say("per-q-head lists, block 128")
    q = normal_bf16(5, "q", (B, 1, Hq, D))
    k = normal_bf16(5, "k", (B, Sk, Hkv, D))
    v = normal_bf16(5, "v", (B, Sk, Hkv, D))
    g = rng(5, "lists")
    n = 5
    idx = np.stack([g.choice(Sk // 128, n, replace=False) for _ in range(B * Hq)]).reshape(B, Hq, 1, n)
    cnt = g.integers(0, n + 1, size=(B, Hq, 1)).astype(np.int32)
    cnt[0, 0, 0] = 0                                              # an empty list: (0, -inf)
    pat = bsa.BlockPattern(dev_i32(cnt), dev_i32(idx), 128, 128)
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, cnt, idx.astype(np.int32), 128, 128)
    check_o(host(o), o_ref, "per-q-head")
    check_lse(host(lse), lse_ref, "per-q-head lse")
    assert np.isneginf(host(lse)[0, 0, 0]) and np.all(host(o)[0, 0, 0] == 0)


@pytest.mark.parametrize("Sq,Sk,D", [(3, 1000, 128), (2, 777, 64), (1, 64, 128)])
def test_dense_ragged_causal(Sq, Sk, D):
    """Dense causal decode with several query positions and a key count off the 64 grid."""
    B, Hq, Hkv = 2, 8, 2
    say("dense ragged causal", Sq, Sk, D)
    q = normal_bf16(6, "q", (B, Sq, Hq, D))
    k = normal_bf16(6, "k", (B, Sk, Hkv, D))
    v = normal_bf16(6, "v", (B, Sk, Hkv, D))
    o, lse = bsa.bsa_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), None, causal=True, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.dense(q, k, v, causal=True)
    check_o(host(o), o_ref, "dense")
    check_lse(host(lse), lse_ref, "dense lse")


def test_broadcast_table_and_determinism():
    """The 1-D block table shared by every head; two runs are bitwise identical."""
    B, Hq, Hkv, D, Sk = 3, 4, 4, 64, 1024
    say("1-D table broadcast")
    q = normal_bf16(8, "q", (B, 1, Hq, D))
    k = normal_bf16(8, "k", (B, Sk, Hkv, D))
    v = normal_bf16(8, "v", (B, Sk, Hkv, D))
    ids = np.array([3, 0, 9, 14, 7], np.int32)
    pat = bsa.BlockPattern.table(dev_i32(ids), 64)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o1, l1 = bsa.bsa_fwd(dq, dk, dv, pat, out_dtype=torch.float32)
    o2, l2 = bsa.bsa_fwd(dq, dk, dv, pat, out_dtype=torch.float32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cnt = np.full((B, Hq, 1), 5, np.int32)
    idx = np.broadcast_to(ids, (B, Hq, 1, 5)).copy()
    o_ref, lse_ref = oracle.block_sparse(q, k, v, cnt, idx, 1, 64)
    check_o(host(o1), o_ref, "table")
    check_lse(host(l1), lse_ref, "table lse")


@pytest.fixture(scope="module")
def spec_full():
    say("generating speculative+sparse decode workload (B=32, Hq=32, Hkv=8, Sk=32768)")
    w = spec_sparse_decode()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


def test_speculative_full_size_every_group(spec_full):
    """Full workload in the benchmark's launch configuration; every (b, kv head) group (all
    1024 query rows) recomputed by the oracle."""
    w = spec_full
    say("speculative+sparse full size")
    s0 = w["spec_start"]
    n = w["missed"].shape[-1]
    missed = bsa.BlockPattern(dev_i32(np.full((32, 8, 1), n, np.int32)), dev_i32(w["missed"][:, :, None, :]), 128, 64)
    o, lse = bsa.speculative_sparse(w["dq"], w["dk"][:, s0:], w["dv"][:, s0:], w["dk"], w["dv"], missed,
                                    out_dtype=torch.float32)
    oh, lh = host(o), host(lse)
    G = 4
    o_ref = np.zeros_like(oh)
    lse_ref = np.zeros_like(lh)
    for b in range(32):
        for hkv in range(8):
            hs = slice(hkv * G, (hkv + 1) * G)
            o_ref[b:b + 1, :, hs], lse_ref[b:b + 1, hs] = oracle.speculative_sparse(
                w["q"][b:b + 1, :, hs], w["k"][b:b + 1, s0:, hkv:hkv + 1], w["v"][b:b + 1, s0:, hkv:hkv + 1],
                w["k"][b:b + 1, :, hkv:hkv + 1], w["v"][b:b + 1, :, hkv:hkv + 1], np.full((1, 1, 1), n, np.int32),
                w["missed"][b:b + 1, hkv:hkv + 1, None, :], 64, causal_spec=True)
    check_o(oh, o_ref, "full size, all 256 groups")
    check_lse(lh, lse_ref, "full size lse, all 256 groups")


@pytest.mark.parametrize("Sq,causal_spec", [(1, True), (8, True), (3, False)])
def test_speculative_partials_and_fallback(Sq, causal_spec):
    """bsa_speculative_partials + bsa_combine equal the oracle's two-pass result, on the fused
    decode launch (Sq*G <= 16) and on the prefill fallback (Sq=8, G=4 gives 32 rows)."""
    B, Hq, Hkv, D, Sk, bs = 2, 8, 2, 128, 2048, 64
    say("speculative partials", Sq, causal_spec)
    q = normal_bf16(9, "q", (B, Sq, Hq, D))
    k = normal_bf16(9, "k", (B, Sk, Hkv, D))
    v = normal_bf16(9, "v", (B, Sk, Hkv, D))
    s0 = Sk - 320                                   # speculative keys: the last 320 (not a 64 multiple)
    g = rng(9, "missed")
    n = 7
    idx = np.stack([np.sort(g.choice(s0 // bs, n, replace=False)) for _ in range(B * Hkv)]).reshape(B, Hkv, 1, n)
    idx = idx.astype(np.int32)
    cnt = np.full((B, Hkv, 1), n, np.int32)
    cnt[1, 0, 0] = 0                                 # one group with nothing missed
    pat = bsa.BlockPattern(dev_i32(cnt), dev_i32(idx), 128, bs)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    op, lp = bsa.bsa_speculative_partials(dq, dk[:, s0:], dv[:, s0:], dk, dv, pat, causal_spec=causal_spec)
    o, lse = bsa.bsa_combine(op, lp, out_dtype=torch.float32)
    o2, lse2 = bsa.speculative_sparse(dq, dk[:, s0:], dv[:, s0:], dk, dv, pat, causal_spec=causal_spec,
                                      out_dtype=torch.float32)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle.speculative_sparse(q, k[:, s0:], v[:, s0:], k, v, cnt, idx, bs, causal_spec=causal_spec)
    check_o(host(o), o_ref, "speculative partials")
    check_lse(host(lse), lse_ref, "speculative partials lse")


@pytest.mark.parametrize("E", [0, 1, 5])
def test_fwd_partials_grouping_decode(E):
    """Partials of E entries each (E = 0: the library's split) recombine to bsa_fwd's result."""
    B, Hq, Hkv, D, Sk = 2, 8, 2, 128, 4096
    say("decode partials E =", E)
    q = normal_bf16(10, "q", (B, 1, Hq, D))
    k = normal_bf16(10, "k", (B, Sk, Hkv, D))
    v = normal_bf16(10, "v", (B, Sk, Hkv, D))
    g = rng(10, "lists")
    n = 23
    idx = np.stack([g.choice(Sk // 64, n, replace=False) for _ in range(B * Hkv)]).reshape(B, Hkv, 1, n)
    idx = idx.astype(np.int32)
    cnt = np.full((B, Hkv, 1), n, np.int32)
    pat = bsa.BlockPattern(dev_i32(cnt), dev_i32(idx), 128, 64)
    op, lp = bsa.bsa_fwd_partials(dev_bf16(q), dev_bf16(k), dev_bf16(v), pat, E)
    assert op.shape[0] == bsa.bsa_num_partials(dev_bf16(q), dev_bf16(k), pat, E)
    o, lse = bsa.bsa_combine(op, lp, out_dtype=torch.float32)
    o_ref, lse_ref = oracle.block_sparse(q, k, v, cnt, idx, 1, 64)
    check_o(host(o), o_ref, f"partials E={E}")
    check_lse(host(lse), lse_ref, f"partials E={E} lse")


def test_graph_replay_matches_eager():
    """The speculative passes and the combine captured in one HIP graph (as the benchmark
    replays a decode step): every replay, with eager work and synchronizations in between,
    equals the eager result bit for bit, and the eager result matches the oracle."""
    w = _small_spec()
    say("graph replay of a speculative decode step")
    q, k, v = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    s0 = w["spec_start"]
    missed, cnt, idx = _pattern_kv(w["missed"], 64, w["Hkv"])
    o_part, lse_part = bsa.bsa_speculative_partials(q, k[:, s0:], v[:, s0:], k, v, missed)
    out = torch.empty((q.shape[0], 1, q.shape[2], q.shape[3]), dtype=torch.float32, device=q.device)
    lse = torch.empty((q.shape[0], q.shape[2], 1), dtype=torch.float32, device=q.device)

    def step():
        bsa.bsa_speculative_partials(q, k[:, s0:], v[:, s0:], k, v, missed, o_part=o_part, lse_part=lse_part)
        bsa.bsa_combine(o_part, lse_part, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    o_eager, l_eager = out.clone(), lse.clone()
    o_ref, lse_ref = oracle.speculative_sparse(w["q"], w["k"][:, s0:], w["v"][:, s0:], w["k"], w["v"], cnt, idx, 64,
                                               causal_spec=True)
    check_o(host(o_eager), o_ref, "eager step")
    check_lse(host(l_eager), lse_ref, "eager step lse")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device=q.device)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager) and torch.equal(lse, l_eager), f"replay {r}"
