"""The solution of A x = b as exact fractions, by fraction-free Bareiss elimination.

Test infrastructure (see ``oracle/__init__``).  Follows the exact-solve card
(phanerozoic/exact-solve): "API" -- an ``[n][c]`` result of exact fractions,
``None`` for a matrix with determinant zero; "Correctness" -- an exact
elimination oracle, and the check that A N = d b holds in integers for the
numerators N over a common denominator d.

The result has a plain definition (x = A^-1 b in lowest terms with a positive
denominator), so this module computes that definition directly and does not
follow the p-adic method at all.  Bareiss (1968) keeps every intermediate an
integer: after step k, entry (i, j) of the trailing block is a (k+1)-by-(k+1)
minor, so each division by the previous pivot is exact.
"""
from __future__ import annotations

from fractions import Fraction
from math import gcd


def _as_int_rows(A):
    return [[int(v) for v in row] for row in A]


def bareiss_eliminate(A, b):
    """Forward Bareiss elimination of [A | b].

    Returns (M, d) with M the n x (n + c) upper-triangular integer array and
    d = M[n-1][n-1] = +-det A, or (None, 0) if A is singular.  Pivot rule:
    the lowest row index at or below k with a nonzero entry in column k.
    """
    A = _as_int_rows(A)
    b = _as_int_rows(b)
    n = len(A)
    c = len(b[0]) if n else 0
    M = [A[i] + b[i] for i in range(n)]
    prev = 1
    for k in range(n):
        piv = next((i for i in range(k, n) if M[i][k] != 0), None)
        if piv is None:
            return None, 0
        if piv != k:
            M[k], M[piv] = M[piv], M[k]
        rk = M[k]
        akk = rk[k]
        for i in range(k + 1, n):
            ri = M[i]
            aik = ri[k]
            for j in range(k + 1, n + c):
                num = akk * ri[j] - aik * rk[j]
                q, r = divmod(num, prev)
                assert r == 0, "Bareiss division must be exact"
                ri[j] = q
            ri[k] = 0
        prev = akk
    return M, M[n - 1][n - 1]


def bareiss_det(A) -> int:
    """det A with its sign by Bareiss elimination (0 when singular).

    Same pivot rule as ``bareiss_eliminate``; each row swap flips the sign.
    """
    M = _as_int_rows(A)
    n = len(M)
    if n == 0:
        return 1
    prev, sign = 1, 1
    for k in range(n):
        piv = next((i for i in range(k, n) if M[i][k] != 0), None)
        if piv is None:
            return 0
        if piv != k:
            M[k], M[piv] = M[piv], M[k]
            sign = -sign
        for i in range(k + 1, n):
            for j in range(k + 1, n):
                q, r = divmod(M[k][k] * M[i][j] - M[i][k] * M[k][j], prev)
                assert r == 0
                M[i][j] = q
            M[i][k] = 0
        prev = M[k][k]
    return sign * M[n - 1][n - 1]


def bareiss_solve_numerators(A, b):
    """Return (N, d): integer numerators N [n][c] with x = N / d, d = +-det A.

    Fraction-free back substitution on the eliminated system: every row of M
    is an integer combination of rows of [A | b], so U x = b' row by row, and
    N_i = d * x_i is an integer by Cramer's rule, making each division exact.
    Returns (None, 0) if A is singular.
    """
    n = len(A)
    M, d = bareiss_eliminate(A, b)
    if M is None:
        return None, 0
    c = len(M[0]) - n
    N = [[0] * c for _ in range(n)]
    for t in range(c):
        for i in range(n - 1, -1, -1):
            s = d * M[i][n + t]
            row = M[i]
            for j in range(i + 1, n):
                s -= row[j] * N[j][t]
            q, r = divmod(s, row[i])
            assert r == 0, "back substitution must be exact"
            N[i][t] = q
    return N, d


def reduce_fraction(num: int, den: int):
    """Lowest terms with a positive denominator; zero is 0/1."""
    assert den != 0
    g = gcd(num, den)
    num //= g
    den //= g
    if den < 0:
        num, den = -num, -den
    return num, den


def check_identity(A, b, N, d) -> bool:
    """A N == d b in exact integer arithmetic (card, "Correctness")."""
    n = len(A)
    c = len(N[0]) if n else 0
    for i in range(n):
        Ai = A[i]
        for t in range(c):
            s = 0
            for j in range(n):
                s += int(Ai[j]) * N[j][t]
            if s != d * int(b[i][t]):
                return False
    return True


def check_solution(A, b, X) -> bool:
    """A x == b exactly for X given as [n][c] of (num, den) pairs."""
    n = len(A)
    c = len(b[0]) if n else 0
    for t in range(c):
        # common denominator of column t
        L = 1
        for i in range(n):
            den = X[i][t][1]
            L = L // gcd(L, den) * den
        Nt = [X[j][t][0] * (L // X[j][t][1]) for j in range(n)]
        for i in range(n):
            s = 0
            Ai = A[i]
            for j in range(n):
                s += int(Ai[j]) * Nt[j]
            if s != L * int(b[i][t]):
                return False
    return True


def solve(A, b):
    """Exact solution x = A^-1 b.

    Returns ``None`` if A is singular over Q, else an ``[n][c]`` list of
    ``(num, den)`` integer pairs in lowest terms with ``den > 0`` (zero is
    ``(0, 1)``).  Every returned solution is checked with A x == b.
    """
    N, d = bareiss_solve_numerators(A, b)
    if N is None:
        return None
    assert check_identity(A, b, N, d)
    return [[reduce_fraction(v, d) for v in row] for row in N]


def solve_fractions(A, b):
    """Same as ``solve`` with ``fractions.Fraction`` entries."""
    X = solve(A, b)
    if X is None:
        return None
    return [[Fraction(p, q) for (p, q) in row] for row in X]
