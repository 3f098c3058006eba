"""Seeded synthetic inputs for the block-Toeplitz FFT matvec.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the GPU path and the CPU oracle can be fed from it.

Workloads follow "Mixed-precision FFTMatvec performance optimization on AMD
GPUs", section 4.1 (single-GPU table at Nm=5000, Nd=100, Nt=1000). The page
gives no value distribution; the one used here is:

  F_k[r, c] = z * exp(-k / tau) / sqrt(Nm),  z ~ N(0, 1) i.i.d.,  tau = Nt / 4
  m[j, c], d[i, r] ~ N(0, 1) i.i.d.

Every block is drawn from its own stream,
``numpy.random.default_rng(SeedSequence([seed, tag]))``, with tag = k for
block F_k, tag = Nt for m and tag = Nt + 1 for d, so a block can be drawn
alone (chunked generation of large operators) and the result does not depend
on how the work is split.

Layouts (row-major, float64):
  F : [Nt][Nd][Nm]   block F_k at F[k]
  m : [Nt][Nm]       m_j, the j-th time step of the input of F
  d : [Nt][Nd]       d_i, the i-th time step of the input of F*
"""

from __future__ import annotations

import math
import os
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Shape:
    name: str
    Nm: int
    Nd: int
    Nt: int

    @property
    def N(self) -> int:
        return 2 * self.Nt

    @property
    def K(self) -> int:
        return self.Nt + 1


TINY = Shape("tiny", Nm=8, Nd=4, Nt=16)
SMALL = Shape("small", Nm=500, Nd=20, Nt=256)
MAIN = Shape("main", Nm=5000, Nd=100, Nt=1000)
SCALE = Shape("scale", Nm=20000, Nd=100, Nt=2000)
SHAPES = {s.name: s for s in (TINY, SMALL, MAIN, SCALE)}


def decay_scale(Nt: int) -> float:
    """tau = Nt / 4 (exp(-k/4) at Nt=16, exp(-k/500) at Nt=2000)."""
    return Nt / 4.0


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag)]))


def block(k: int, Nm: int, Nd: int, Nt: int, seed: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Block F_k as an [Nd][Nm] float64 array."""
    if out is None:
        out = np.empty((Nd, Nm), dtype=np.float64)
    _rng(seed, k).standard_normal(out=out)
    out *= math.exp(-k / decay_scale(Nt)) / math.sqrt(Nm)
    return out


def operator(Nm: int, Nd: int, Nt: int, seed: int = 0, out: np.ndarray | None = None,
             workers: int | None = None) -> np.ndarray:
    """All blocks, F [Nt][Nd][Nm] float64.

    ``out`` may be any writable float64 array of that shape (e.g. pinned
    host memory).  With ``workers`` > 1 the blocks are drawn by that many
    threads; the values are the same either way.
    """
    if out is None:
        out = np.empty((Nt, Nd, Nm), dtype=np.float64)
    assert out.shape == (Nt, Nd, Nm) and out.dtype == np.float64
    if workers is None:
        workers = 1 if Nt * Nd * Nm < 50_000_000 else min(16, os.cpu_count() or 1)
    if workers <= 1:
        for k in range(Nt):
            block(k, Nm, Nd, Nt, seed, out=out[k])
        return out
    _operator_parallel(out, Nm, Nd, Nt, seed, workers)
    return out


def _operator_parallel(out, Nm, Nd, Nt, seed, workers):
    """Blocks drawn by a pool of threads straight into ``out`` (numpy's
    generator and the scaling release the GIL for bulk fills). Threads, not
    processes: nothing is forked or executed, which matters when the calling
    process has already initialised a GPU (a profiler can do that before the
    program starts)."""
    from concurrent.futures import ThreadPoolExecutor

    step = max(1, -(-Nt // (4 * workers)))

    def fill(k0):
        for k in range(k0, min(Nt, k0 + step)):
            block(k, Nm, Nd, Nt, seed, out=out[k])

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(0, Nt, step)))


def input_m(Nm: int, Nt: int, seed: int = 0) -> np.ndarray:
    """m [Nt][Nm] float64, i.i.d. N(0, 1), tag = Nt."""
    return _rng(seed, Nt).standard_normal((Nt, Nm))


def input_d(Nd: int, Nt: int, seed: int = 0) -> np.ndarray:
    """d [Nt][Nd] float64, i.i.d. N(0, 1), tag = Nt + 1."""
    return _rng(seed, Nt + 1).standard_normal((Nt, Nd))


def problem(shape: Shape, seed: int = 0, workers: int | None = None):
    """(F, m, d) for a named shape."""
    F = operator(shape.Nm, shape.Nd, shape.Nt, seed, workers=workers)
    return F, input_m(shape.Nm, shape.Nt, seed), input_d(shape.Nd, shape.Nt, seed)
