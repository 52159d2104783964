"""The stored full-size expectations (tests/golden/full_size.npz, written by
tests/golden/make_full_size.py from the float64 oracle) against the oracle itself, on a part
the CPU redoes in seconds: one (sequence, head) row of the vertical-slash conversion (its
digest) and the gate thresholds of sampled query blocks, recomputed from the oracle's tile
maxima, plus the properties the parity tests rely on (every threshold at least 1e-2 from every
tile maximum of its row, about half of the off-diagonal tiles skipped)."""
import os

import numpy as np
import pytest

import oracle
from synth.workloads import gated_prefill, thresholds_from_tile_max, vs_varlen_prefill
from tests.golden.make_full_size import GATE, VS, _vs_row, _W, vs_digest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "full_size.npz")


@pytest.fixture(scope="module")
def gold():
    return np.load(GOLDEN, allow_pickle=False)


def test_vs_digest_of_one_row(gold):
    _W["vs"] = vs_varlen_prefill(seqlens=VS["seqlens"], H=VS["H"], nnz_v=VS["nnz_v"], nnz_s=VS["nnz_s"],
                                 block=VS["block"], context_size=VS["context"], with_tensors=False)
    try:
        b, h, d = _vs_row((1, 7))
    finally:
        _W.clear()
    assert d.encode() == gold["vs_sha"][1, 7]
    assert len(set(gold["vs_sha"].ravel().tolist())) == gold["vs_sha"].size   # rows differ from each other


def test_vs_digest_sees_a_changed_entry():
    bc = np.array([2, 0], np.int32)
    bo = np.array([[5, 70], [0, 0]], np.int32)
    cc = np.array([1, 0], np.int32)
    ci = np.array([[3], [0]], np.int32)
    d0 = vs_digest(bc, bo, cc, ci)
    bo2 = bo.copy()
    bo2[0, 1] = 71
    assert vs_digest(bc, bo2, cc, ci) != d0
    bo3 = bo.copy()
    bo3[1, 0] = 9          # past the count: not part of the result
    assert vs_digest(bc, bo3, cc, ci) == d0


def test_gate_thresholds_of_sampled_blocks(gold):
    w = gated_prefill(S=GATE["S"], Hq=GATE["Hq"])
    T = gold["gate_T"]
    assert T.shape == (32, 512) and np.isneginf(T[:, 0]).all() and np.isfinite(T[:, 1:]).all()
    for h, i in [(0, 1), (3, 77), (31, 300), (12, 511)]:
        t = oracle.tile_max_row(w["q"], w["k"], 0, h, i, GATE["tile"], GATE["tile"])
        assert T[h, i] == np.float32(thresholds_from_tile_max(t, i))
        assert np.abs(t[:i].astype(np.float32) - T[h, i]).min() >= 1e-2 - 1e-6
    assert 0.45 < float(gold["skip_frac"]) < 0.55
