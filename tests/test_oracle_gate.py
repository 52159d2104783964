"""Pins for the oracle's BSFA gating: special thresholds, library tile maxima, equivalence
with block-sparse attention over the kept tiles, and the threshold generator's margin."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f64, normal_bf16
from synth.workloads import gated_prefill, thresholds_from_tile_max

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _small(seed=21, S=256, Hq=4, Hkv=2, D=32, bs=32):
    w = gated_prefill(seed=seed, B=1, Hq=Hq, Hkv=Hkv, S=S, D=D, bs=bs)
    return w["q"], w["k"], w["v"], bs


def _median_thresholds(q, k, bs):
    S, Hq = q.shape[1], q.shape[2]
    nqb = S // bs
    T = np.zeros((1, Hq, nqb), np.float32)
    for h in range(Hq):
        for i in range(nqb):
            T[0, h, i] = thresholds_from_tile_max(oracle.tile_max_row(q, k, 0, h, i, bs, bs), i)
    return T


def _sdpa(q, k, v, mask=None, causal=False):
    tq, tk, tv = (torch.from_numpy(bf16_to_f64(x)).permute(0, 2, 1, 3) for x in (q, k, v))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal,
                                                         enable_gqa=tq.shape[1] != tk.shape[1])
    return o.permute(0, 2, 1, 3).numpy()


def test_minus_inf_threshold_is_dense_causal():
    q, k, v, bs = _small()
    nqb = q.shape[1] // bs
    T = np.full((1, q.shape[2], nqb), -np.inf, np.float32)
    o, lse, keep, _ = oracle.gated(q, k, v, T, bs, bs)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), atol=1e-12)
    assert np.array_equal(keep[0, 0], np.tril(np.ones((nqb, nqb), np.uint8)))


def test_plus_inf_threshold_is_block_diagonal_causal():
    q, k, v, bs = _small()
    S, nqb = q.shape[1], q.shape[1] // bs
    T = np.full((1, q.shape[2], nqb), np.inf, np.float32)
    o, _, keep, _ = oracle.gated(q, k, v, T, bs, bs)
    blockdiag = np.kron(np.eye(nqb, dtype=bool), np.ones((bs, bs), bool)) & np.tril(np.ones((S, S), bool))
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask=blockdiag), atol=1e-12)
    assert np.array_equal(keep[0, 1], np.eye(nqb, dtype=np.uint8))


def test_tile_max_matches_max_pool_and_keep_rule():
    """Tile maxima from torch max_pool2d over the causally masked score matrix."""
    q, k, v, bs = _small(seed=22)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    nqb = S // bs
    g = np.random.default_rng(0)
    T = g.normal(1.0, 1.0, size=(1, Hq, nqb)).astype(np.float32)
    _, _, keep, tmax = oracle.gated(q, k, v, T, bs, bs)
    qf, kf = bf16_to_f64(q), bf16_to_f64(k)
    for h in range(Hq):
        s = qf[0, :, h] @ kf[0, :, h // (Hq // Hkv)].T / math.sqrt(D)
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        pooled = torch.nn.functional.max_pool2d(torch.from_numpy(s)[None, None], bs)[0, 0].numpy()
        lower = np.tril(np.ones((nqb, nqb), bool))
        np.testing.assert_allclose(tmax[0, h][lower], pooled[lower], rtol=0, atol=1e-12)
        want = ((pooled.astype(np.float32) >= T[0, h][:, None]) | np.eye(nqb, dtype=bool)) & lower
        assert np.array_equal(keep[0, h].astype(bool), want)


def test_gated_equals_block_sparse_on_kept_tiles():
    q, k, v, bs = _small(seed=23)
    B, S, Hq, _ = q.shape
    nqb = S // bs
    T = _median_thresholds(q, k, bs)
    o, lse, keep, _ = oracle.gated(q, k, v, T, bs, bs)
    count = keep.sum(-1).astype(np.int32)
    index = np.zeros((1, Hq, nqb, nqb), np.int32)
    for h in range(Hq):
        for i in range(nqb):
            kept = np.nonzero(keep[0, h, i])[0]
            index[0, h, i, :kept.size] = kept
    ob, lb = oracle.block_sparse(q, k, v, count, index, bs, bs, causal=True)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)
    assert 0 < keep.sum() < np.tril(np.ones((nqb, nqb))).sum() * Hq


def test_gated_rows_match_full():
    q, k, v, bs = _small(seed=24)
    S, Hq = q.shape[1], q.shape[2]
    nqb = S // bs
    T = _median_thresholds(q, k, bs)
    o, lse, keep, tmax = oracle.gated(q, k, v, T, bs, bs)
    for h, i, rows in [(0, 0, [0, 5, 31]), (3, 5, [160, 170, 191]), (2, 7, [224, 255])]:
        orow, lrow, kr, t = oracle.gated_rows(q, k, v, T[0, h, i], 0, h, i, rows, bs, bs)
        np.testing.assert_allclose(orow, o[0, rows, h], atol=1e-12)
        np.testing.assert_allclose(lrow, lse[0, h, rows], atol=1e-12)
        assert np.array_equal(kr, keep[0, h, i, :i + 1])
        np.testing.assert_allclose(t, tmax[0, h, i, :i + 1], atol=1e-12)


def test_threshold_generator_margin_and_rate():
    q, k, v, bs = _small(seed=25, S=1024, Hq=2, Hkv=1, D=64, bs=64)
    nqb = q.shape[1] // bs
    skipped = total = 0
    for h in range(2):
        for i in range(nqb):
            t = oracle.tile_max_row(q, k, 0, h, i, bs, bs)
            T = thresholds_from_tile_max(t, i)
            if i == 0:
                assert T == -np.inf
                continue
            assert np.min(np.abs(t[:i] - T)) >= 1e-2 - 1e-6
            skipped += int(np.sum(t[:i] < T))
            total += i
    assert 0.3 < skipped / total < 0.7


# ---- threshold calibration ----

@pytest.mark.parametrize("k_keep", [1, 3, 6])
def test_calibrated_threshold_keeps_exactly_k_per_row(k_keep):
    """Gating a calibration sample with its own thresholds keeps min(k, i) off-diagonal tiles
    of each query block i (the maxima of these inputs are distinct), so the realised density is
    the target one.  Checked through the gated oracle's own keep rule."""
    q, k, v, bs = _small(seed=31)
    T, per = oracle.calibrate(q, k, k_keep, bs, bs)
    assert np.array_equal(T, per[0])
    nqb = T.shape[1]
    assert np.isneginf(T[:, :k_keep]).all() and np.isfinite(T[:, k_keep:]).all()
    _, _, keep, tmax = oracle.gated(q, k, v, T[None].astype(np.float32), bs, bs)
    for h in range(T.shape[0]):
        for i in range(nqb):
            off = tmax[0, h, i, :i]
            assert np.unique(off.astype(np.float32)).size == off.size
            assert keep[0, h, i, :i].sum() == min(k_keep, i), (h, i)
            assert keep[0, h, i, i] == 1
    realised, target = oracle.gated_density(keep, k_keep)
    assert abs(realised - target) < 1e-12
    assert abs(target - sum(min(k_keep, i) + 1 for i in range(nqb)) / (nqb * (nqb + 1) / 2)) < 1e-12


def test_calibration_averages_samples():
    """Two samples, the second with every query doubled (exact in bf16): its scores, and so its
    k-th largest tile maximum, double; the calibrated threshold is the mean, 1.5x the first."""
    from synth import f32_to_bf16_bits
    q, k, _, bs = _small(seed=32)
    q2 = f32_to_bf16_bits((2.0 * bf16_to_f64(q)).astype(np.float32))
    qq = np.concatenate([q, q2])
    kk = np.concatenate([k, k])
    T, per = oracle.calibrate(qq, kk, 2, bs, bs)
    fin = np.isfinite(per[0])
    np.testing.assert_allclose(per[1][fin], 2.0 * per[0][fin], rtol=1e-12)
    np.testing.assert_allclose(T[fin], 1.5 * per[0][fin], rtol=1e-12)
    assert np.isneginf(T[~fin]).all() and (~fin).sum() == 2 * T.shape[0]


def test_calibration_with_k_past_every_row_keeps_everything():
    q, k, v, bs = _small(seed=33, S=128)
    T, _ = oracle.calibrate(q, k, 4, bs, bs)
    assert np.isneginf(T).all()
    _, _, keep, _ = oracle.gated(q, k, v, T[None].astype(np.float32), bs, bs)
    realised, target = oracle.gated_density(keep, 4)
    assert realised == 1.0 and target == 1.0
    with pytest.raises(ValueError):
        oracle.calibrate(q, k, 0, bs, bs)


# ---- the "count" reading of a skipped tile (scores kept in the maximum and normaliser) ----

def _dense_causal_lse(q, k):
    """log-sum-exp of the scaled causal scores, by torch.logsumexp in float64 (independent of
    the oracle's softmax)."""
    qf, kf = bf16_to_f64(q), bf16_to_f64(k)
    B, S, Hq, D = qf.shape
    G = Hq // kf.shape[2]
    out = np.zeros((B, Hq, S))
    for h in range(Hq):
        s = torch.from_numpy(qf[0, :, h] @ kf[0, :, h // G].T / math.sqrt(D))
        s = s.masked_fill(~torch.from_numpy(np.tril(np.ones((S, S), bool))), float("-inf"))
        out[0, h] = torch.logsumexp(s, dim=-1).numpy()
    return out


def test_count_reading_has_the_dense_causal_lse():
    """Every causal score stays in the normaliser, whatever the thresholds."""
    q, k, v, bs = _small(seed=24)
    want = _dense_causal_lse(q, k)
    for T in (_median_thresholds(q, k, bs), np.full((1, q.shape[2], q.shape[1] // bs), np.inf, np.float32)):
        _, lse, _, _ = oracle.gated(q, k, v, T, bs, bs, skipped="count")
        np.testing.assert_allclose(lse, want, atol=1e-11, rtol=0)


def test_count_and_drop_share_the_numerator():
    """O exp(LSE) is the sum of exp(score) v over the kept keys under both readings; the keep
    decisions are the same."""
    q, k, v, bs = _small(seed=25)
    T = _median_thresholds(q, k, bs)
    od, ld, kd, _ = oracle.gated(q, k, v, T, bs, bs, skipped="drop")
    oc, lc, kc, _ = oracle.gated(q, k, v, T, bs, bs, skipped="count")
    assert np.array_equal(kd, kc)
    assert (kd[0][:, np.tril(np.ones(kd.shape[-2:], bool), -1)] == 0).any()   # some tiles are skipped
    np.testing.assert_allclose(oc * np.exp(lc)[..., None].transpose(0, 2, 1, 3),
                               od * np.exp(ld)[..., None].transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)
    assert np.abs(oc - od).max() > 1e-3          # the readings do differ where tiles are skipped


def test_count_reading_with_constant_values_gives_the_kept_mass():
    """V = c on every key: O = c times the share of the causal mass in kept tiles, i.e.
    c exp(LSE over kept tiles - dense causal LSE)."""
    q, k, v, bs = _small(seed=26)
    c = 0.75
    v1 = np.full_like(v, np.uint16(0x3F40))      # bf16 bits of 0.75
    T = _median_thresholds(q, k, bs)
    oc, _, _, _ = oracle.gated(q, k, v1, T, bs, bs, skipped="count")
    _, ld, _, _ = oracle.gated(q, k, v1, T, bs, bs, skipped="drop")
    share = np.exp(ld - _dense_causal_lse(q, k))                  # [B, Hq, S]
    np.testing.assert_allclose(oc, c * share.transpose(0, 2, 1)[..., None] * np.ones(oc.shape), rtol=1e-10,
                               atol=1e-13)


def test_count_reading_with_minus_inf_threshold_is_dense_causal():
    q, k, v, bs = _small(seed=27)
    T = np.full((1, q.shape[2], q.shape[1] // bs), -np.inf, np.float32)
    o, _, _, _ = oracle.gated(q, k, v, T, bs, bs, skipped="count")
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), atol=1e-12)


def test_gated_rows_count_matches_gated():
    q, k, v, bs = _small(seed=28)
    T = _median_thresholds(q, k, bs)
    o, lse, _, _ = oracle.gated(q, k, v, T, bs, bs, skipped="count")
    for h, i in [(0, 3), (3, 7), (1, 0)]:
        rows = np.arange(i * bs, (i + 1) * bs)
        orr, lr, _, _ = oracle.gated_rows(q, k, v, T[0, h, i], 0, h, i, rows, bs, bs, skipped="count")
        np.testing.assert_allclose(orr, o[0, rows, h], atol=1e-12)
        np.testing.assert_allclose(lr, lse[0, h, rows], atol=1e-12)
