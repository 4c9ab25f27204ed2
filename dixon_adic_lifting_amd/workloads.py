"""Seeded synthetic inputs for the exact solver and its oracle.

This module only draws and lays out integers.  It holds none of the solver's
arithmetic (no residues, no elimination, no lifting) so that both sides of a
parity test -- the HIP path and the CPU oracle -- can take their inputs from
here without sharing any of the method.

Workloads follow the exact-solve card (phanerozoic/exact-solve, sections
"Usage", "Measured" and "Correctness"): integer ``A`` of shape ``[n, n]`` and
``b`` of shape ``[n, c]``; the timed cases draw entries of 24 bits; the
correctness systems are the order-30 symmetric Pascal matrix, systems built
around a chosen integer solution, and Hilbert matrices scaled to integers.

Generator: ``numpy.random.default_rng(seed)`` (PCG64); ``integers(lo, hi)``
with ``hi`` exclusive; ``A`` is drawn row-major first, then ``b`` as ``[n][c]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

INT24_LO = -(1 << 23)
INT24_HI = 1 << 23


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    c: int
    kind: str          # "uniform" or "pascal"
    a_lo: int = 0      # inclusive
    a_hi: int = 0      # exclusive
    b_lo: int = 0
    b_hi: int = 0
    seed: int = 0


# The five configurations: a tiny 8-bit system, the order-30 Pascal system,
# and the card's 24-bit shapes (n = 256 and 1024 with one right-hand side)
# plus a 16-column system at n = 2048.
WORKLOADS = {
    "c1_n32_int8": Workload("c1_n32_int8", 32, 1, "uniform", -128, 128, -(1 << 20), 1 << 20, 1),
    "c2_pascal30": Workload("c2_pascal30", 30, 1, "pascal", 0, 0, -(1 << 20), 1 << 20, 2),
    "c3_n256_int24": Workload("c3_n256_int24", 256, 1, "uniform", INT24_LO, INT24_HI, INT24_LO, INT24_HI, 3),
    "c4_n1024_int24": Workload("c4_n1024_int24", 1024, 1, "uniform", INT24_LO, INT24_HI, INT24_LO, INT24_HI, 4),
    "c5_n2048_c16_int24": Workload("c5_n2048_c16_int24", 2048, 16, "uniform", INT24_LO, INT24_HI, INT24_LO, INT24_HI, 5),
}

# The card's other measured shapes (24-bit entries), for sweeps.
CARD_SHAPES = [(128, 1), (256, 1), (512, 1), (1024, 1), (256, 16), (512, 16)]


def pascal_matrix(n: int) -> np.ndarray:
    """Symmetric Pascal matrix S[i][j] = C(i + j, i), 0-indexed, as int64."""
    S = np.empty((n, n), dtype=np.int64)
    for i in range(n):
        for j in range(n):
            S[i, j] = math.comb(i + j, i)
    return S


def generate(w: Workload | str, attempt: int = 0):
    """Return (A, b) as C-contiguous int64 numpy arrays for a workload.

    ``attempt`` selects a redraw (seed + 1000 * attempt) for callers that must
    reject a singular draw; attempt 0 is the canonical input.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed + 1000 * attempt)
    if w.kind == "pascal":
        A = pascal_matrix(w.n)
    else:
        A = rng.integers(w.a_lo, w.a_hi, size=(w.n, w.n), dtype=np.int64)
    b = rng.integers(w.b_lo, w.b_hi, size=(w.n, w.c), dtype=np.int64)
    return np.ascontiguousarray(A), np.ascontiguousarray(b)


def uniform_system(n: int, c: int, bits: int, seed: int):
    """A and b i.i.d. uniform signed ``bits``-bit integers, seeded."""
    lo, hi = -(1 << (bits - 1)), 1 << (bits - 1)
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi, size=(n, n), dtype=np.int64)
    b = rng.integers(lo, hi, size=(n, c), dtype=np.int64)
    return np.ascontiguousarray(A), np.ascontiguousarray(b)


def planted_system(n: int, c: int, a_bits: int, x_bits: int, seed: int):
    """A uniform, integer solution X planted, b = A @ X (must fit int64).

    Returns (A, b, X).  Bounds are chosen by the caller so that
    n * 2^(a_bits-1) * 2^(x_bits-1) < 2^63.
    """
    assert n * (1 << (a_bits - 1)) * (1 << (x_bits - 1)) < (1 << 63)
    rng = np.random.default_rng(seed)
    A = rng.integers(-(1 << (a_bits - 1)), 1 << (a_bits - 1), size=(n, n), dtype=np.int64)
    X = rng.integers(-(1 << (x_bits - 1)), 1 << (x_bits - 1), size=(n, c), dtype=np.int64)
    b = np.array([[sum(int(A[i, k]) * int(X[k, t]) for k in range(n)) for t in range(c)]
                  for i in range(n)], dtype=np.int64)
    return np.ascontiguousarray(A), np.ascontiguousarray(b), X


def scaled_hilbert(n: int):
    """A[i][j] = L / (i + j + 1) with L = lcm(1, ..., 2n - 1), 0-indexed.

    Integral and dense in denominators; fits the range limit for n <= 21.
    """
    L = 1
    for k in range(1, 2 * n):
        L = L * k // math.gcd(L, k)
    A = np.array([[L // (i + j + 1) for j in range(n)] for i in range(n)], dtype=np.int64)
    return A, L


def duplicate_row_system(n: int, seed: int):
    """Singular family: row n-1 repeats row 0."""
    A, b = uniform_system(n, 1, 16, seed)
    A[n - 1] = A[0]
    return A, b


def zero_column_system(n: int, seed: int):
    """Singular family: column n // 2 is zero."""
    A, b = uniform_system(n, 1, 16, seed)
    A[:, n // 2] = 0
    return A, b


def low_rank_system(n: int, rank: int, seed: int):
    """Singular family: A = U V with U [n, rank], V [rank, n] small integers."""
    rng = np.random.default_rng(seed)
    U = rng.integers(-8, 8, size=(n, rank), dtype=np.int64)
    V = rng.integers(-8, 8, size=(rank, n), dtype=np.int64)
    A = U @ V
    b = rng.integers(-(1 << 20), 1 << 20, size=(n, 1), dtype=np.int64)
    return np.ascontiguousarray(A), b
