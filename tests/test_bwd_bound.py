"""The backward's per-element error bound (tests/bwd_bound.py) holds for an emulation of the
kernels' arithmetic on the CPU: float32 products and sums, P and dS rounded to bf16 before the
products that use them, the row dot D taken from an O rounded to bf16.  The emulation's error
against the float64 oracle stays inside the bound everywhere, and is not far below it
everywhere (the bound is not vacuous)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f64, normal_bf16
from tests.bwd_bound import grad_bounds

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _emulate(q, k, v, do, mask, scale, o_used):
    q, k, v, do = (np.asarray(x, np.float32) for x in (q, k, v, do))
    s = np.where(mask, (q @ k.T) * np.float32(scale), -np.inf).astype(np.float32)
    m = s.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True, dtype=np.float32))
    p = np.exp(s - lse).astype(np.float32)
    pb = _bf16(p)
    dv = pb.T @ do
    dp = do @ v.T
    d = (do * np.asarray(o_used, np.float32)).sum(axis=1, keepdims=True, dtype=np.float32)
    dsb = _bf16(p * (dp - d))
    return np.float32(scale) * (dsb @ k), np.float32(scale) * (dsb.T @ q), dv


@pytest.mark.parametrize("Sq,Sk,causal", [(128, 256, True), (96, 200, False)])
def test_emulated_kernel_arithmetic_stays_within_the_bound(Sq, Sk, causal):
    D = 128
    q, k, v, do = (bf16_to_f64(normal_bf16(61, t, (1, n, 1, D))) for t, n in (("q", Sq), ("k", Sk), ("v", Sk), ("do", Sq)))
    scale = 1.0 / math.sqrt(D)
    mask = oracle.causal_mask(Sq, Sk) if causal else np.ones((Sq, Sk), bool)
    o64, _ = oracle.dense(q, k, v, causal=causal)
    o_used = _bf16(o64)                       # the forward's O handed over in bf16
    rq, rk, rv = oracle.block_sparse_bwd(q, k, v, do, causal=causal)
    eq, ek, ev = _emulate(q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0], mask, scale, o_used[0, :, 0])
    bq, bk, bv = grad_bounds(q, k, v, do, o_used.astype(np.float64), lambda b, h: mask)
    for name, e, r, bd in (("dq", eq, rq[0, :, 0], bq[0, :, 0]), ("dk", ek, rk[0, :, 0], bk[0, :, 0]),
                           ("dv", ev, rv[0, :, 0], bv[0, :, 0])):
        err = np.abs(e - r)
        assert (err <= bd + 1e-7).all(), (name, float((err - bd).max()))
        assert float((err / (bd + 1e-7)).max()) > 0.02, name    # the bound is within 50x of the error
