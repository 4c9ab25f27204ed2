"""Dixon p-adic lifting written out on Python integers -- TEST INFRASTRUCTURE.

Follows the exact-solve card (phanerozoic/exact-solve), section "Method", in
its order and notation:

* modulus P = prod(q_j), a squarefree product of odd primes q_j < 256;
* B = A^-1 mod P, r_0 = b, x_i = B r_i mod P, r_{i+1} = (r_i - A x_i) / P;
* m digits suffice once P^m is larger than 2 N D, N and D being the
  Hadamard-type bounds on the numerators and on the denominator;
* the rational reconstruction finds the denominator shared by the
  components from a few of them, then each numerator by a single product
  modulo P^m.

Readings where the card is silent (each also listed with the design notes):
the digits are balanced, x_i in [-(P-1)/2, (P-1)/2]; primes that divide det A
are dropped from P; the bound is P^m > 2 N D with D the Hadamard bound on
|det A| and N the Cramer-Hadamard bound on every numerator; the sample is
the first four components in row-major order.
"""
from __future__ import annotations

from math import gcd, isqrt, prod

from .modular import inverse_mod


def _ceil_sqrt(s: int) -> int:
    return 0 if s == 0 else isqrt(s - 1) + 1


def hadamard_bounds(A, b):
    """Integer upper bounds (N, D) with |det A| <= D and |det A_i^t| <= N.

    D = min(prod of row 2-norms, prod of column 2-norms) of A.  A_i^t is A with
    column i replaced by column t of b (Cramer's rule: x_i = det A_i^t / det A),
    so N = max_t ||b_t|| * prod_j ||A_j|| / min_j ||A_j|| over columns A_j.
    Every 2-norm is rounded up to an integer, which keeps both bounds valid.
    """
    n = len(A)
    c = len(b[0])
    rows = [_ceil_sqrt(sum(int(v) * int(v) for v in A[i])) for i in range(n)]
    cols = [_ceil_sqrt(sum(int(A[i][j]) ** 2 for i in range(n))) for j in range(n)]
    bcols = [_ceil_sqrt(sum(int(b[i][t]) ** 2 for i in range(n))) for t in range(c)]
    D = min(prod(rows), prod(cols))
    cmin = min(cols)
    Ncol = prod(cols) // cmin if cmin else prod(sorted(cols)[1:])
    N = max(bcols) * Ncol
    return N, D


def step_count(P: int, N: int, D: int) -> int:
    """Least m with P^m > 2 N D."""
    m, Pm = 0, 1
    while Pm <= 2 * N * D:
        m += 1
        Pm *= P
    return m


def surviving_primes(A, primes):
    """Primes q for which A is invertible mod q, and their inverses."""
    live, invs = [], []
    for q in primes:
        Bq = inverse_mod(A, q)
        if Bq is not None:
            live.append(q)
            invs.append(Bq)
    return live, invs


def crt_matrix(invs, primes):
    """B mod P from the per-prime inverses by the Chinese remainder theorem."""
    P = prod(primes)
    n = invs[0].shape[0]
    B = [[0] * n for _ in range(n)]
    for Bq, q in zip(invs, primes):
        Pq = P // q
        e = Pq * pow(Pq % q, -1, q)          # e = 1 mod q, 0 mod the others
        for i in range(n):
            row = B[i]
            src = Bq[i]
            for j in range(n):
                row[j] += int(src[j]) * e
    for i in range(n):
        B[i] = [v % P for v in B[i]]
    return B


def balanced_mod(v: int, P: int) -> int:
    r = v % P
    return r - P if r > (P - 1) // 2 else r


def padic_digits(A, b, primes, m, B=None):
    """The first m Dixon digits for x = A^-1 b over the modulus prod(primes).

    Returns (digits, residuals): digits[i][r][t] = x_i (balanced), residuals[i]
    = r_i as [n][c] Python ints (residuals[0] = b, m + 1 entries).  Every
    division by P is checked to be exact.
    """
    n = len(A)
    c = len(b[0])
    P = prod(primes)
    if B is None:
        _, invs = surviving_primes(A, primes)
        assert len(invs) == len(primes), "A must be invertible modulo every prime"
        B = crt_matrix(invs, primes)
    Ai = [[int(v) for v in row] for row in A]
    r = [[int(b[i][t]) for t in range(c)] for i in range(n)]
    digits, residuals = [], [r]
    for _ in range(m):
        x = [[balanced_mod(sum(B[i][j] * r[j][t] for j in range(n)), P) for t in range(c)]
             for i in range(n)]
        nr = [[0] * c for _ in range(n)]
        for i in range(n):
            for t in range(c):
                s = r[i][t] - sum(Ai[i][j] * x[j][t] for j in range(n))
                q, rem = divmod(s, P)
                assert rem == 0, "r_i - A x_i must be divisible by P"
                nr[i][t] = q
        digits.append(x)
        residuals.append(nr)
        r = nr
    return digits, residuals


def assemble(digits, P: int):
    """X = sum_i x_i P^i per component, as Python ints (may be negative)."""
    m = len(digits)
    n = len(digits[0])
    c = len(digits[0][0])
    X = [[0] * c for _ in range(n)]
    for i in range(m - 1, -1, -1):
        for r in range(n):
            for t in range(c):
                X[r][t] = X[r][t] * P + digits[i][r][t]
    return X


def rational_reconstruct(a: int, M: int, N: int, D: int):
    """Wang's rational reconstruction: the unique n/d = a mod M, |n| <= N, 0 < d <= D.

    Extended Euclid on (M, a mod M) stops at the first remainder <= N; the
    matching cofactor is the denominator.  Requires 2 N D < M.  Returns
    (num, den) in lowest terms with den > 0, or None if no such fraction.
    """
    r0, r1 = M, a % M
    t0, t1 = 0, 1
    while r1 > N:
        q = r0 // r1
        r0, r1 = r1, r0 - q * r1
        t0, t1 = t1, t0 - q * t1
    if t1 == 0 or abs(t1) > D or gcd(r1, abs(t1)) != 1:
        return None
    if t1 < 0:
        return -r1, -t1
    return r1, t1


SAMPLE_SIZE = 4


def sample_indices(total: int):
    """Components whose reconstructed denominators form the common
    denominator.  The card asks only for a few sampled components; the
    plainest reading is the first few in row-major order, here four.  The
    result does not depend on the choice: a component whose numerator falls
    outside the bound is reconstructed on its own and widens d."""
    return list(range(min(total, SAMPLE_SIZE)))


def reconstruct_solution(X, M: int, N: int, D: int):
    """Rational solution from X = A^-1 b mod M (M > 2 N D).

    Common denominator d = lcm of the sampled components' reconstructed
    denominators; then for each component y = d X mods M.  If |y| <= N the
    component is y / d (in lowest terms), otherwise it is reconstructed on its
    own and d takes the lcm with its denominator.
    """
    n = len(X)
    c = len(X[0])
    flat = [X[r][t] for r in range(n) for t in range(c)]
    d = 1
    for idx in sample_indices(len(flat)):
        f = rational_reconstruct(flat[idx], M, N, D)
        if f is None:
            return None
        d = d * f[1] // gcd(d, f[1])
    out = []
    for v in flat:
        y = balanced_mod(d * v, M)
        if abs(y) <= N:
            g = gcd(y, d)
            out.append((y // g, d // g))
        else:
            f = rational_reconstruct(v, M, N, D)
            if f is None:
                return None
            out.append(f)
            d = d * f[1] // gcd(d, f[1])
    return [out[r * c:(r + 1) * c] for r in range(n)]


def dixon_solve(A, b, primes):
    """Whole method on Python integers: inverse, digits, reconstruction.

    Returns (solution or None, info) with info = dict(live=..., m=..., N=..., D=...).
    Primes that divide det A are dropped from the modulus.
    """
    live, invs = surviving_primes(A, primes)
    if not live:
        return None, {"live": []}
    P = prod(live)
    N, D = hadamard_bounds(A, b)
    m = step_count(P, N, D)
    B = crt_matrix(invs, live)
    digits, _ = padic_digits(A, b, live, m, B=B)
    X = assemble(digits, P)
    sol = reconstruct_solution(X, P ** m, N, D)
    return sol, {"live": live, "m": m, "N": N, "D": D, "P": P}
