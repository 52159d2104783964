"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
import sys

import numpy as np
import torch

from synth import to_torch_bf16

O_TOL = 1e-2      # max-abs on O (float32 output), bf16 inputs with float32 accumulation
LSE_TOL = 1e-3    # max-abs on LSE


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return to_torch_bf16(bits).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, what: str, bf16_out: bool = False):
    """max-abs on O; for a bf16 output the bound adds half a bf16 ulp of the reference."""
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    tol = O_TOL
    if bf16_out:
        mag = np.maximum(np.abs(o_ref), 1e-30)
        tol = O_TOL + 2.0 ** (np.floor(np.log2(mag)) - 8)
    bad = err > tol
    assert not bad.any(), f"{what}: max |dO| = {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    print(f"[parity] {what}: max |dO| = {err.max():.3e}", flush=True)
    return float(err.max())


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str):
    assert lse_gpu.shape == lse_ref.shape
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), inf_ref), f"{what}: -inf pattern differs"
    fin = ~inf_ref
    if fin.any():
        err = np.abs(lse_gpu[fin] - lse_ref[fin])
        assert err.max() <= LSE_TOL, f"{what}: max |dLSE| = {err.max():.3e}"
        print(f"[parity] {what}: max |dLSE| = {err.max():.3e}", flush=True)
        return float(err.max())
    return 0.0
