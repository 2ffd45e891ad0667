"""Seeded dense operands (features, edge values, Q/K/V).

Large arrays are filled in fixed-size blocks, block b drawing from
``SeedSequence(seed).spawn(n_blocks)[b]`` with PCG64, so the values depend only
on the seed and the shape, never on the number of threads used to fill them.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_BLOCK = 1 << 22  # elements per independently seeded block


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(shape, seed: int, draw) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n = out.size
    nb = max(1, -(-n // _BLOCK))
    seqs = np.random.SeedSequence(seed).spawn(nb)

    def work(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(seqs[b]))
        draw(g, out[lo:hi])

    if nb == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nb)))
    return out.reshape(shape)


def dense_normal(shape, seed: int) -> np.ndarray:
    """fp32 N(0, 1)."""
    return _fill(shape, seed, lambda g, o: g.standard_normal(out=o, dtype=np.float32))


def dense_uniform(shape, seed: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """fp32 U(lo, hi)."""

    def draw(g, o):
        g.random(out=o, dtype=np.float32)
        if lo != 0.0 or hi != 1.0:
            o *= np.float32(hi - lo)
            o += np.float32(lo)

    return _fill(shape, seed, draw)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even) and return the raw
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
