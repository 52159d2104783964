"""GPU parity for BSFA gated prefill: keep masks bit-exact, tile maxima, O and LSE, at small
size (every row) and at full size (every keep decision of all 32 heads; tile maxima, O and LSE
on sampled query blocks), with thresholds from the oracle's exact tile maxima at least 1e-2
from every tile maximum."""
import os

import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth.workloads import gated_prefill, thresholds_from_tile_max
from tests.golden.make_full_size import keep_digest
from tests.gpu_util import check_lse, check_o, dev_bf16, host, say

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_size.npz")

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def small():
    w = gated_prefill(seed=41, B=2, Hq=4, Hkv=2, S=1024, D=128, bs=128)
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    nqb = 8
    T = np.zeros((2, 4, nqb), np.float32)
    for b in range(2):
        for h in range(4):
            for i in range(nqb):
                T[b, h, i] = thresholds_from_tile_max(oracle.tile_max_row(w["q"], w["k"], b, h, i, 128, 128), i)
    w["T"] = T
    return w


@pytest.mark.parametrize("skipped", ["drop", "count"])
@pytest.mark.parametrize("mode", ["median", "-inf", "+inf"])
def test_gated_small(small, mode, skipped):
    w = small
    say("gated small", mode, skipped)
    T = {"median": w["T"], "-inf": np.full_like(w["T"], -np.inf), "+inf": np.full_like(w["T"], np.inf)}[mode]
    o, lse, keep, tmax = bsa.bsa_fwd_gated(w["dq"], w["dk"], w["dv"], torch.from_numpy(T).cuda(), skipped=skipped,
                                           out_dtype=torch.float32, return_tile_max=True)
    o_ref, lse_ref, keep_ref, tmax_ref = oracle.gated(w["q"], w["k"], w["v"], T, 128, 128, skipped=skipped)
    lower = np.tril(np.ones((8, 8), bool))
    kg = keep.cpu().numpy()
    assert np.array_equal(kg[..., lower], keep_ref[..., lower]), "keep mask differs"
    tg = tmax.cpu().numpy().astype(np.float64)
    assert np.abs(tg[..., lower] - tmax_ref[..., lower]).max() < 1e-3
    check_o(host(o), o_ref, f"gated {mode} {skipped}")
    check_lse(host(lse), lse_ref, f"gated {mode} {skipped} lse")
    if mode == "median":
        off = lower & ~np.eye(8, dtype=bool)
        frac = 1.0 - kg[..., off].mean()
        assert 0.3 < frac < 0.7, frac


def test_gated_matches_block_sparse_path(small):
    """The gated result equals the block-sparse kernel on the kept tiles.  Both are GPU paths,
    each within the parity tolerance of the oracle (checked above), with independent bf16
    rounding of P (different tile orders): they agree to twice that tolerance."""
    w = small
    say("gated vs block-sparse path")
    o, lse, keep, _ = bsa.bsa_fwd_gated(w["dq"], w["dk"], w["dv"], torch.from_numpy(w["T"]).cuda(),
                                        out_dtype=torch.float32)
    kg = keep.cpu().numpy()
    count = kg.sum(-1).astype(np.int32)
    index = np.zeros_like(kg, dtype=np.int32)
    for b in range(2):
        for h in range(4):
            for i in range(8):
                kept = np.nonzero(kg[b, h, i, :i + 1])[0]
                index[b, h, i, :kept.size] = kept
    pat = bsa.BlockPattern(torch.from_numpy(count).cuda(), torch.from_numpy(index).cuda(), 128, 128)
    ob, lb = bsa.bsa_fwd(w["dq"], w["dk"], w["dv"], pat, causal=True, out_dtype=torch.float32)
    diff = np.abs(host(o) - host(ob)).max()
    assert diff <= 2 * 1e-2, diff
    check_lse(host(lse), host(lb), "gated vs block path lse")


@pytest.fixture(scope="module")
def cfg4():
    say("generating gated prefill workload (S=65536, Hq=32, Hkv=8)")
    w = gated_prefill()
    w["dq"], w["dk"], w["dv"] = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    return w


def test_gated_full_size_every_keep_decision(cfg4):
    """The benchmark's gate at full size: thresholds for all 16,384 (head, query block) rows from
    the oracle's float64 tile maxima (gap midpoints at least 1e-2 from every maximum, nearest a
    50% split; stored by tests/golden/make_full_size.py), keep masks of all 32 heads compared bit
    for bit with the oracle's (by digest), tile maxima of sampled rows, and O / LSE on every row
    of sampled query blocks."""
    w = cfg4
    gold = np.load(GOLDEN, allow_pickle=False)
    T = gold["gate_T"][None].astype(np.float32)
    say("gated full size at the oracle's thresholds")
    o, lse, keep, tmax = bsa.bsa_fwd_gated(w["dq"], w["dk"], w["dv"], torch.from_numpy(T).cuda(),
                                           out_dtype=torch.float32, return_tile_max=True)
    kg = keep.cpu().numpy()
    tg = tmax.cpu().numpy().astype(np.float64)
    bad = [h for h in range(32) if keep_digest(kg[0, h]).encode() != gold["keep_sha"][h]]
    if bad:
        h = bad[0]
        for i in range(512):
            t = oracle.tile_max_row(w["q"], w["k"], 0, h, i, 128, 128)
            kr = (t.astype(np.float32) >= T[0, h, i]).astype(np.uint8)
            kr[i] = 1
            assert np.array_equal(kg[0, h, i, :i + 1], kr), f"keep mask differs at h={h} i={i}"
        raise AssertionError(f"keep digests differ for heads {bad}")
    lower = np.tril(np.ones((512, 512), bool), -1)
    skip = 1.0 - float(kg[0][:, lower].mean())
    assert abs(skip - float(gold["skip_frac"])) < 1e-12
    print(f"[parity] gated full size: keep masks of 32 heads bit-exact, skip fraction {skip:.4f}", flush=True)
    oh, lh = host(o), host(lse)
    say("gated full size, skipped tiles counted in the normaliser")
    oc, lc, kc, _ = bsa.bsa_fwd_gated(w["dq"], w["dk"], w["dv"], torch.from_numpy(T).cuda(), skipped="count",
                                      out_dtype=torch.float32)
    assert torch.equal(kc, keep), "the keep decisions do not depend on the skipped-tile reading"
    och, lch = host(oc), host(lc)
    for h, i in [(0, 511), (31, 300), (9, 1), (17, 64), (5, 0), (22, 450), (12, 127), (28, 2)]:
        rows = np.arange(i * 128, (i + 1) * 128)
        o_ref, lse_ref, kr, t = oracle.gated_rows(w["q"], w["k"], w["v"], T[0, h, i], 0, h, i, rows, 128, 128)
        assert np.array_equal(kg[0, h, i, :i + 1], kr), f"keep mask differs h={h} i={i}"
        assert np.abs(tg[0, h, i, :i + 1] - t).max() < 1e-3, f"tile maxima h={h} i={i}"
        if i:
            assert np.abs(t[:i].astype(np.float32) - T[0, h, i]).min() >= 1e-2 - 1e-6
        check_o(oh[0, rows, h], o_ref, f"gated full h={h} i={i}")
        check_lse(lh[0, h, rows], lse_ref, f"gated full lse h={h} i={i}")
        o_ref, lse_ref, _, _ = oracle.gated_rows(w["q"], w["k"], w["v"], T[0, h, i], 0, h, i, rows, 128, 128,
                                                 skipped="count")
        check_o(och[0, rows, h], o_ref, f"gated full (count) h={h} i={i}")
        check_lse(lch[0, h, rows], lse_ref, f"gated full (count) lse h={h} i={i}")


# ---- threshold calibration ----

@pytest.mark.parametrize("k_keep", [1, 3, 7])
def test_calibrate_small(small, k_keep):
    """Tile maxima (j <= i) and thresholds against the oracle over two calibration samples;
    k_keep = 7 leaves only the last query block with a finite threshold."""
    w = small
    say("calibrate small", k_keep)
    T, tmax = bsa.bsfa_calibrate(w["dq"], w["dk"], k_keep)
    T_ref, per_ref = oracle.calibrate(w["q"], w["k"], k_keep, 128, 128)
    lower = np.tril(np.ones((8, 8), bool))
    tg = tmax.cpu().numpy().astype(np.float64)
    for b in range(2):
        for h in range(4):
            for i in range(8):
                t = oracle.tile_max_row(w["q"], w["k"], b, h, i, 128, 128)
                assert np.abs(tg[b, h, i, :i + 1] - t).max() < 1e-3, (b, h, i)
    assert np.isnan(tg[..., ~lower]).all(), "entries above the diagonal must stay untouched"
    Tg = T.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(Tg), np.isneginf(T_ref))
    fin = np.isfinite(T_ref)
    assert np.abs(Tg[fin] - T_ref[fin]).max() < 1e-3


def test_calibrated_gate_keeps_k_per_row(small):
    """One calibration sample gated with its own thresholds keeps exactly min(k, i) off-diagonal
    tiles per query block: the thresholds are that sample's own tile maxima, computed by the
    same tile loop, so the comparison is exact.  The realised density then equals the target."""
    w = small
    k_keep = 3
    say("calibrated gate keeps k per row")
    q0, k0, v0 = w["dq"][:1], w["dk"][:1], w["dv"][:1]
    T, tmax = bsa.bsfa_calibrate(q0, k0, k_keep)
    _, _, keep, tmax2 = bsa.bsa_fwd_gated(q0, k0, v0, T, out_dtype=torch.float32, return_tile_max=True)
    kg = keep.cpu().numpy()
    lower = np.tril(np.ones((8, 8), bool))
    assert np.array_equal(tmax.cpu().numpy()[..., lower], tmax2.cpu().numpy()[..., lower])
    for h in range(4):
        for i in range(8):
            assert kg[0, h, i, :i].sum() == min(k_keep, i) and kg[0, h, i, i] == 1, (h, i)
    realised, target = oracle.gated_density(kg, k_keep)
    assert realised == target


def test_calibrate_full_size_sampled(cfg4):
    """Thresholds at the full 65536-token shape, k = 64, on sampled rows."""
    w = cfg4
    say("calibrate full size")
    T, tmax = bsa.bsfa_calibrate(w["dq"], w["dk"], 64)
    Tg = T.cpu().numpy().astype(np.float64)
    tg = tmax.cpu().numpy()
    assert np.isneginf(Tg[:, :64]).all() and np.isfinite(Tg[:, 64:]).all()
    for h, i in [(0, 511), (31, 300), (17, 64), (8, 65), (3, 200)]:
        say("oracle tile maxima", h, i)
        t = oracle.tile_max_row(w["q"], w["k"], 0, h, i, 128, 128)
        assert np.abs(tg[0, h, i, :i + 1] - t).max() < 1e-3, (h, i)
        want = np.sort(t[:i])[::-1][63]
        assert abs(Tg[h, i] - want) < 1e-3, (h, i, Tg[h, i], want)
