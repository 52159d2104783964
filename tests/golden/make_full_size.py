"""Writes tests/golden/full_size.npz: expected values for the full-size parity tests that the
float64 oracle takes minutes to produce, computed here once by the oracle alone.

  vs_sha     [2, 32] sha256 digests, one per (sequence, head), of the vertical-slash
             conversion of the vertical-slash workload (seqlens 65536 + 32768, 32 heads,
             1000 vertical + 2000 slash indices, blocks 64, context 65536): for every query
             block m in order, block_count, the block_count valid block_offset entries,
             column_count and the column_count valid column_index entries, as little-endian
             int32 (``vs_digest``).
  gate_T     [32, 512] float32 thresholds of the gated workload (S = 65536, 32 query heads,
             128x128 tiles), picked per query block from the oracle's float64 tile maxima
             with ``synth.workloads.thresholds_from_tile_max`` (the gap midpoint at least
             1e-2 from every tile maximum, nearest a 50% split; -inf for block 0).
  keep_sha   [32] sha256 digests, one per head, of the oracle's keep decisions at those
             thresholds: the lower triangle (j <= i) of the [512, 512] keep mask as uint8,
             row by row (``keep_digest``).
  skip_frac  float64: the fraction of off-diagonal causal tiles those decisions skip.

Run from the repository root:  python tests/golden/make_full_size.py  (about 3 minutes on 8
cores).  Only ``synth`` (seeded inputs) and ``oracle`` are used.
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "full_size.npz")

VS = dict(seqlens=(65536, 32768), H=32, nnz_v=1000, nnz_s=2000, block=64, context=65536)
GATE = dict(S=65536, Hq=32, tile=128)


def vs_digest(bc, bo, cc, ci) -> str:
    """Digest of one (sequence, head) row of conversion output: per query block, the counts and
    the valid prefixes (entries past a count are unspecified and left out)."""
    h = hashlib.sha256()
    for m in range(bc.shape[0]):
        nb, nc = int(bc[m]), int(cc[m])
        h.update(np.asarray([nb], "<i4").tobytes())
        h.update(np.ascontiguousarray(bo[m, :nb], "<i4").tobytes())
        h.update(np.asarray([nc], "<i4").tobytes())
        h.update(np.ascontiguousarray(ci[m, :nc], "<i4").tobytes())
    return h.hexdigest()


def keep_digest(keep) -> str:
    """Digest of one head's keep mask [nQB, nKB]: the lower triangle (j <= i) as uint8, row by row."""
    keep = np.asarray(keep)
    lower = np.tril(np.ones(keep.shape, bool))
    return hashlib.sha256(np.ascontiguousarray(keep[lower], np.uint8).tobytes()).hexdigest()


_W = {}


def _vs_row(bh):
    import oracle

    w = _W["vs"]
    b, h = bh
    L = int(w["seqlens"][b])
    R = (VS["context"] + VS["block"] - 1) // VS["block"]
    bc = np.zeros(R, np.int32)
    cc = np.zeros(R, np.int32)
    bo = np.zeros((R, VS["nnz_s"]), np.int32)
    ci = np.zeros((R, VS["nnz_v"]), np.int32)
    for m in range(R):
        wins, cols = oracle.vs_convert_item(L, L, w["vertical"][b, h], w["slash"][b, h], m, VS["block"], VS["block"])
        bc[m], cc[m] = len(wins), len(cols)
        bo[m, :len(wins)] = wins
        ci[m, :len(cols)] = cols
    return b, h, vs_digest(bc, bo, cc, ci)


def _gate_head(h):
    import oracle
    from synth.workloads import thresholds_from_tile_max

    w = _W["gate"]
    nqb = GATE["S"] // GATE["tile"]
    T = np.zeros(nqb, np.float32)
    keep = np.zeros((nqb, nqb), np.uint8)
    for i in range(nqb):
        t = oracle.tile_max_row(w["q"], w["k"], 0, h, i, GATE["tile"], GATE["tile"])
        T[i] = thresholds_from_tile_max(t, i)
        keep[i, :i + 1] = (t.astype(np.float32) >= T[i]).astype(np.uint8)
        keep[i, i] = 1
    off = np.tril(np.ones((nqb, nqb), bool), -1)
    return h, T, keep_digest(keep), int(keep[off].sum()), int(off.sum())


def _init():
    from threadpoolctl import threadpool_limits

    global _LIMIT
    _LIMIT = threadpool_limits(limits=1)


def main():
    from synth.workloads import gated_prefill, vs_varlen_prefill

    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("fork")
    t0 = time.time()
    _W["vs"] = vs_varlen_prefill(seqlens=VS["seqlens"], H=VS["H"], nnz_v=VS["nnz_v"], nnz_s=VS["nnz_s"],
                                 block=VS["block"], context_size=VS["context"], with_tensors=False)
    vs_sha = np.zeros((len(VS["seqlens"]), VS["H"]), "S64")
    with ctx.Pool(procs, initializer=_init) as pool:
        for b, h, d in pool.imap_unordered(_vs_row, [(b, h) for b in range(len(VS["seqlens"])) for h in range(VS["H"])]):
            vs_sha[b, h] = d.encode()
    print(f"vertical-slash conversion digests: {time.time() - t0:.0f} s", flush=True)

    t0 = time.time()
    _W["gate"] = gated_prefill(S=GATE["S"], Hq=GATE["Hq"])
    nqb = GATE["S"] // GATE["tile"]
    gate_T = np.zeros((GATE["Hq"], nqb), np.float32)
    keep_sha = np.zeros(GATE["Hq"], "S64")
    skipped = total = 0
    with ctx.Pool(procs, initializer=_init) as pool:
        for h, T, d, kept, off in pool.imap_unordered(_gate_head, range(GATE["Hq"])):
            gate_T[h] = T
            keep_sha[h] = d.encode()
            skipped += off - kept
            total += off
            print(f"  gate head {h}: {kept}/{off} off-diagonal tiles kept", flush=True)
    print(f"gate thresholds and keep digests: {time.time() - t0:.0f} s", flush=True)
    np.savez(OUT, vs_sha=vs_sha, gate_T=gate_T, keep_sha=keep_sha, skip_frac=np.float64(skipped / total))
    print(f"wrote {OUT} (skip fraction {skipped / total:.4f})")


if __name__ == "__main__":
    main()
