"""Primes below 256 and A^-1 mod q by plain Gauss-Jordan -- TEST INFRASTRUCTURE.

Follows the exact-solve card (phanerozoic/exact-solve), section "Method": the
modulus is a squarefree product of primes below 256 and must be odd, and the
GPU computes A^-1 mod q for every prime by Gauss-Jordan elimination over the
augmented matrix [A | I].  Here that is written out per prime with numpy
row operations (a library primitive for each whole-row update), nothing
fused or blocked.
"""
from __future__ import annotations

import numpy as np


def odd_primes_below(bound: int = 256):
    """Odd primes q < bound by trial division (3, 5, 7, ..., 251 for 256)."""
    out = []
    for v in range(3, bound, 2):
        if all(v % d for d in range(3, int(v ** 0.5) + 1, 2)):
            out.append(v)
    return out


def inverse_mod(A, q: int):
    """A^-1 mod q as an int64 array with entries in [0, q), or None.

    Gauss-Jordan on [A | I] mod q: for each column k pick the lowest row at or
    below k whose entry is nonzero mod q, swap it up, scale it to a unit
    pivot, and clear column k from every other row.  No pivot means A is
    singular mod q (equivalently q divides det A) and None is returned.
    """
    A = np.asarray(A, dtype=object)
    n = A.shape[0]
    M = np.zeros((n, 2 * n), dtype=np.int64)
    for i in range(n):
        for j in range(n):
            M[i, j] = int(A[i, j]) % q
        M[i, n + i] = 1
    for k in range(n):
        nz = np.nonzero(M[k:, k])[0]
        if nz.size == 0:
            return None
        p = k + int(nz[0])
        if p != k:
            M[[k, p]] = M[[p, k]]
        inv = pow(int(M[k, k]), -1, q)
        M[k] = (M[k] * inv) % q
        f = M[:, k].copy()
        f[k] = 0
        M = (M - np.outer(f, M[k])) % q
    return np.ascontiguousarray(M[:, n:])


def det_mod(A, q: int) -> int:
    """det A mod q by Gaussian elimination mod q (in [0, q))."""
    M = np.array([[int(v) % q for v in row] for row in np.asarray(A, dtype=object)],
                 dtype=np.int64)
    n = M.shape[0]
    det = 1
    for k in range(n):
        nz = np.nonzero(M[k:, k])[0]
        if nz.size == 0:
            return 0
        p = k + int(nz[0])
        if p != k:
            M[[k, p]] = M[[p, k]]
            det = -det
        det = (det * int(M[k, k])) % q
        inv = pow(int(M[k, k]), -1, q)
        f = (M[k + 1:, k] * inv) % q
        M[k + 1:] = (M[k + 1:] - np.outer(f, M[k])) % q
    return det % q
