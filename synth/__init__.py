"""Seeded synthetic inputs for the block-sparse attention workloads.

This is test and benchmark infrastructure shared by the CPU oracle checks and
the GPU path.  It draws random numbers, encodes them as bfloat16 bit patterns
and builds index lists.  It performs none of the attention arithmetic: no
dot products, softmax, maxima of scores or index conversion live here.

Every array is a deterministic function of (seed, tag): a tensor is drawn in
fixed chunks of ``CHUNK`` elements, chunk ``c`` from child ``c`` of
``numpy.random.SeedSequence([seed, tag])`` with the PCG64 bit generator, so the
result does not depend on how many threads draw it.

bf16 tensors are returned as ``numpy.uint16`` bit patterns.  ``bf16_to_f64``
widens them exactly; ``to_torch_bf16`` reinterprets them for upload.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _tag(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the upper 16 bits of the rounded float32 pattern as uint16.  The
    inputs here are finite normal draws, so NaN handling is not needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def to_torch_bf16(bits: np.ndarray):
    """View uint16 bf16 bit patterns as a CPU ``torch.bfloat16`` tensor (no copy)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def normal_f32(seed: int, tag: str, shape) -> np.ndarray:
    """Standard normal float32 draws of ``shape``, chunked and multi-threaded."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = np.random.SeedSequence([seed, _tag(tag)]).spawn(max(nchunks, 1))

    def fill(c: int) -> None:
        g = np.random.Generator(np.random.PCG64(kids[c]))
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normal_bf16(seed: int, tag: str, shape) -> np.ndarray:
    """Standard normal draws rounded to bf16 bit patterns."""
    x = normal_f32(seed, tag, shape)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for lo in range(0, flat.size, step):
        out[lo:lo + step] = f32_to_bf16_bits(flat[lo:lo + step])
    return out.reshape(shape)


def rng(seed: int, tag: str) -> np.random.Generator:
    """A single PCG64 stream for small draws (index lists, scales)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _tag(tag)])))


# ---------------------------------------------------------------------------
# Index lists
# ---------------------------------------------------------------------------

def random_subset_sorted(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """k distinct integers from [0, n), ascending."""
    return np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)


def power_law_unique(g: np.random.Generator, L: int, n: int, force_zero: bool = True) -> np.ndarray:
    """n distinct integers on [0, L) with p(x) proportional to (x+1)^-2.

    Continuous inverse CDF of the truncated density, floored to an integer;
    repeats are rejected (the first n distinct values in draw order are
    kept).  With ``force_zero`` the value 0 is always included.
    """
    n = min(n, L)
    c = 1.0 - 1.0 / (L + 1.0)
    draws = [np.zeros(1, dtype=np.int64)] if force_zero else []
    batch = max(4096, n * n // 4)
    while True:
        u = g.random(batch)
        x = np.floor(1.0 / (1.0 - u * c) - 1.0).astype(np.int64)
        draws.append(np.clip(x, 0, L - 1))
        allx = np.concatenate(draws)
        _, first = np.unique(allx, return_index=True)
        if first.size >= n:
            order = np.sort(first)[:n]
            return allx[order].astype(np.int32)
        batch *= 2
