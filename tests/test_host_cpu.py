"""CPU tests of the HIP library's host side (no GPU needed).

* every function declared in include/*.h is exported by libexact_solve.so;
* the host big-integer routines agree with Python integers;
* Wang reconstruction agrees with the oracle's;
* the host reconstruction stage (es_reconstruct), fed with the oracle's own
  Dixon digits, returns exactly the oracle's Bareiss solution.
"""
import ctypes
import glob
import math
import os
import random
import re

import numpy as np
import pytest

from dixon_adic_lifting_amd import _lib
from dixon_adic_lifting_amd import workloads as W
import dixon_adic_lifting_amd as es
from oracle import dixon, exact, modular

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lib():
    return _lib.load()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(es_\w+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "es_solve_device" in names and "es_batched_inverse" in names
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name
    assert set(_lib.EXPORTS) <= set(names)


def test_workspace_bytes_limits():
    assert es.workspace_bytes(0, 1) == 0
    assert es.workspace_bytes(1, 0) == 0
    assert es.workspace_bytes((1 << 17) + 1, 1) == 0
    assert es.workspace_bytes(1, 1) > 0
    assert es.workspace_bytes(1024, 1) < es.workspace_bytes(2048, 16)


def test_workspace_bytes_same_on_every_thread():
    """The size query depends on (n, c) only: the same on other threads,
    also after one of them caps the lift's record steps."""
    import threading
    shapes = [(1, 1), (32, 1), (300, 2), (1024, 1), (2048, 16)]
    ref = [es.workspace_bytes(n, c) for n, c in shapes]
    got = {}

    def worker(k, cap):
        lib = _lib.load()
        if cap:
            assert lib.es_set_lift_record_steps(cap) == 0
        got[k] = [es.workspace_bytes(n, c) for n, c in shapes]
        if cap:
            lib.es_set_lift_record_steps(0)

    threads = [threading.Thread(target=worker, args=(k, cap)) for k, cap in enumerate([0, 3, 1, 0])]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(v == ref for v in got.values()) and len(got) == 4


def test_primes_and_strerror():
    assert es.primes() == modular.odd_primes_below(256)
    for st in (0, 1, -1, -2, -3, -4, -5, -6):
        assert _lib.strerror(st)


def test_round_up_reciprocal_gives_exact_quotients():
    """The Gauss-Jordan step divides x = s + f v < 2^16 by q with no
    correction: 256 x times ceil(2^24 / q), high 32 bits of the product, is
    floor(x / q) for every x < 2^16 and every odd prime q < 256 (the
    round-up reciprocal with 16 + 8 bits of precision).  Checked
    exhaustively."""
    x = np.arange(1 << 16, dtype=np.uint64)
    for q in es.primes():
        mq = -(-(1 << 24) // q)
        assert mq < (1 << 24)
        t = ((x << np.uint64(8)) * np.uint64(mq)) >> np.uint64(32)
        assert np.array_equal(t, x // np.uint64(q)), q
        assert int(x[-1] << np.uint64(8)) < (1 << 24)


def test_single_precision_rounding_gives_balanced_residues():
    """The rank-32 updates reduce |x| < 2^19 (32 products of balanced
    residues plus one) as x - t q with t = rint(float(x) * float(1 / q)):
    the float product is within 2^-4 / q of x / q and x / q (q odd) is at
    least 1 / (2q) from every half-integer, so t is the nearest integer and
    x - t q the balanced residue.  Checked exhaustively in IEEE single
    precision (one rounding for 1 / q, one for the product)."""
    x = np.arange(-(1 << 19) + 1, 1 << 19, dtype=np.int64)
    xf = x.astype(np.float32)
    for q in es.primes():
        rq = np.float32(1.0) / np.float32(q)
        t = np.rint((xf * rq).astype(np.float32)).astype(np.int64)
        assert np.abs(t).max() < (1 << 23)  # a signed 24-bit operand
        assert np.array_equal(x - t * q, ((x + q // 2) % q) - q // 2), q


# ------------------------------------------------------------------ bignum

def to_limbs(v):
    v = abs(v)
    out = []
    while v:
        out.append(v & ((1 << 64) - 1))
        v >>= 64
    return out


def arr(limbs):
    a = (ctypes.c_uint64 * max(1, len(limbs)))(*limbs)
    return a, len(limbs)


def from_limbs(buf, n, neg=0):
    v = 0
    for i in range(n - 1, -1, -1):
        v = (v << 64) | buf[i]
    return -v if neg else v


def dbg(op, a, b, cap=8192):
    L = ctypes.CDLL(_lib.LIB_PATH)
    f = L.es_dbg_bignum
    pa, la = arr(to_limbs(a))
    pb, lb = arr(to_limbs(b))
    r1 = (ctypes.c_uint64 * cap)()
    r2 = (ctypes.c_uint64 * cap)()
    l1, l2, n1, n2 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int(), ctypes.c_int()
    st = f(op, pa, la, int(a < 0), pb, lb, int(b < 0), r1, ctypes.byref(l1), ctypes.byref(n1),
           r2, ctypes.byref(l2), ctypes.byref(n2), cap)
    assert st == 0
    return from_limbs(r1, l1.value, n1.value), from_limbs(r2, l2.value, n2.value)


def rand_int(rng, limbs, signed=True):
    v = rng.getrandbits(64 * limbs) if limbs else 0
    # sprinkle in all-ones limbs to stress carries
    if limbs and rng.random() < 0.3:
        v |= ((1 << 64) - 1) << (64 * rng.randrange(limbs))
    return -v if signed and rng.random() < 0.5 else v


SIZES = [0, 1, 2, 3, 7, 39, 40, 41, 64, 100, 257, 700]


@pytest.mark.parametrize("la", SIZES)
def test_bignum_mul(la):
    rng = random.Random(la)
    for lb in [0, 1, 5, 40, 41, 80, 300, 700]:
        a, b = rand_int(rng, la), rand_int(rng, lb)
        assert dbg(0, a, b)[0] == a * b


@pytest.mark.parametrize("la", [1, 2, 5, 40, 90, 400, 1000])
def test_bignum_divmod(la):
    rng = random.Random(100 + la)
    for lb in [1, 2, 3, 17, 64, 200, 500]:
        a, b = rand_int(rng, la), rand_int(rng, lb)
        if b == 0:
            continue
        q, r = dbg(1, a, b)
        tq = abs(a) // abs(b) * (1 if (a < 0) == (b < 0) else -1)
        assert q == tq and r == a - tq * b
    # quotient digit edge cases: divisor with top limb all ones, dividend = k*b - 1
    b = ((1 << 64) - 1) << 128 | 12345
    for k in [1, 2, (1 << 64) - 1, 1 << 70]:
        a = k * b - 1
        q, r = dbg(1, a, b)
        assert (q, r) == (a // b, a % b)


def test_bignum_gcd():
    rng = random.Random(5)
    for la, lb in [(1, 1), (2, 1), (5, 5), (50, 48), (400, 400), (437, 300)]:
        g = rand_int(rng, rng.randrange(1, 4), signed=False) | 1
        a, b = rand_int(rng, la) * g, rand_int(rng, lb) * g
        assert dbg(2, a, b)[0] == math.gcd(a, b)
    assert dbg(2, 0, 0)[0] == 0
    assert dbg(2, 12, 0)[0] == 12
    fib = [1, 1]
    while len(fib) < 3000:
        fib.append(fib[-1] + fib[-2])
    assert dbg(2, fib[-1], fib[-2])[0] == 1   # worst case for Euclid
    # lengths far apart, quotients of 2^100 (a full division) and of 2^61
    # (one in-place step), equal values, powers of two, a large shared factor
    big = rand_int(rng, 300, signed=False) | 1
    cases = [(rand_int(rng, 900, signed=False), rand_int(rng, 3, signed=False) | 1),
             (big * ((1 << 100) + 7) + 3, big), (big * ((1 << 61) + 5) + 11, big),
             (big, big), (1 << 5000, 1 << 3001), ((1 << 4000) * 3, (1 << 4100) * 9),
             (big * rand_int(rng, 600, signed=False), big * rand_int(rng, 580, signed=False))]
    for a, b in cases:
        assert dbg(2, a, b)[0] == math.gcd(a, b)
        assert dbg(2, b, a)[0] == math.gcd(a, b)


def test_bignum_add_sub():
    rng = random.Random(9)
    for _ in range(200):
        a, b = rand_int(rng, rng.randrange(0, 9)), rand_int(rng, rng.randrange(0, 9))
        assert dbg(3, a, b)[0] == a + b
        assert dbg(4, a, b)[0] == a - b


def test_divexact_one_word():
    rng = random.Random(9)
    for la in [0, 1, 2, 5, 40, 300]:
        for _ in range(6):
            a = rand_int(rng, la)
            b = rng.getrandbits(64) >> rng.randrange(64) or 1
            if rng.random() < 0.3:
                b = (b << rng.randrange(8)) % (1 << 64) or 2
            assert dbg(5, a * b, b)[0] == a
    # powers of two (a shift), signed quotients, and limb-boundary shifts
    for la in [0, 1, 2, 7, 300]:
        for t in [0, 1, 6, 31, 63]:
            a = rand_int(rng, la)
            for sgn in (1, -1):
                assert dbg(5, sgn * a << t, 1 << t)[0] == sgn * a
    # not exact, or b wider than one limb: refused
    L = ctypes.CDLL(_lib.LIB_PATH)
    for a, b in [(7, 2), (3 << 70, 1 << 65), (10, 0), ((1 << 200) + 32, 64), ((1 << 100) + 1, 2), (10, 3),
                 ((1 << 300) + 5, 7), (3 * ((1 << 200) + 1) + 1, 3 << 5)]:
        pa, la_ = arr(to_limbs(a))
        pb, lb_ = arr(to_limbs(b))
        r = (ctypes.c_uint64 * 64)()
        l1, n1 = ctypes.c_int32(), ctypes.c_int()
        st = L.es_dbg_bignum(5, pa, la_, 0, pb, lb_, 0, r, ctypes.byref(l1), ctypes.byref(n1), r,
                             ctypes.byref(l1), ctypes.byref(n1), 64)
        assert st != 0


@pytest.mark.parametrize("m,count,parts", [(1, 1, 1), (7, 2, 1), (40, 3, 4), (172, 2, 4), (172, 1, 8), (61, 2, 2)])
def test_assemble_in_parts(m, count, parts):
    """The sample's X = sum_i x_i P^i from balanced digits (384-bit two's
    complement, |x_i| <= P / 2), assembled whole and in `parts` ranges on
    the pool's threads joined pairwise (ranges too short for the split fall
    back to whole components): both against Python's own sum."""
    rng = random.Random(m * 31 + count * 7 + parts)
    P = 1
    for q in modular.odd_primes_below(256):
        P *= q
    digits = np.zeros((count, m, 6), dtype=np.int64)
    want = []
    for k in range(count):
        X = 0
        for i in range(m):
            x = rng.randrange(-(P // 2), P // 2 + 1)
            if rng.random() < 0.1:
                x = rng.choice([0, P // 2, -(P // 2)])
            X += x * P ** i
            u = x % (1 << 384)
            digits[k, i] = np.array([(u >> (64 * t)) & ((1 << 64) - 1) for t in range(6)], dtype=np.uint64).view(np.int64)
        want.append(X)
    L = ctypes.CDLL(_lib.LIB_PATH)
    pP, lP = arr(to_limbs(P))
    cap = 6 * m + 8
    out = (ctypes.c_uint64 * (cap * count))()
    lens = (ctypes.c_int32 * count)()
    neg = (ctypes.c_int * count)()
    st = L.es_dbg_assemble(pP, lP, digits.ctypes.data_as(ctypes.c_void_p), m, count, parts, out, lens, neg, cap)
    assert st == 0, st
    for k in range(count):
        got = from_limbs(out[k * cap:(k + 1) * cap], lens[k], neg[k])
        assert got == want[k], k


def ratrec(a, M, N, D, cap=4096):
    L = ctypes.CDLL(_lib.LIB_PATH)
    args = []
    keep = []
    for v in (a, M, N, D):
        p, ln = arr(to_limbs(v))
        keep.append(p)
        args += [p, ln]
    num = (ctypes.c_uint64 * cap)()
    den = (ctypes.c_uint64 * cap)()
    ln_, ld_, nn = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int()
    st = L.es_dbg_ratrec(*args, num, ctypes.byref(ln_), ctypes.byref(nn), den, ctypes.byref(ld_), cap)
    assert st in (0, 1)
    if st == 1:
        return None
    return from_limbs(num, ln_.value, nn.value), from_limbs(den, ld_.value)


def test_ratrec_matches_oracle():
    rng = random.Random(3)
    P = math.prod(modular.odd_primes_below(256))
    # k = 50: M has more than 256 limbs, so the second run (cofactor updates on
    # a second thread) takes that path; both runs must agree (the hook checks)
    for k in [1, 2, 8, 40, 50]:
        M = P ** k
        half = (M.bit_length() - 2) // 2
        for _ in range(12):
            den = rng.randrange(1, 1 << half)
            num = rng.randrange(-(1 << half), 1 << half)
            if math.gcd(den, M) != 1:
                continue
            a = num * pow(den, -1, M) % M
            expect = dixon.rational_reconstruct(a, M, 1 << half, 1 << half)
            assert ratrec(a, M, 1 << half, 1 << half) == expect
        # a random residue usually has no small fraction
        a = rng.randrange(M)
        assert ratrec(a, M, 1 << half, 1 << half) == dixon.rational_reconstruct(a, M, 1 << half, 1 << half)


@pytest.mark.parametrize("k", [100, 172])
def test_ratrec_long_remainders(k):
    """Moduli of 550 and 860 limbs (the size of the sample's reconstructions
    at n = 1024): the two-word Lehmer matrices over long remainders, with the
    cofactors on a second thread in the hook's second run; both runs must
    agree with the oracle, for balanced and unbalanced bounds (Wang's
    stopping point in the middle, low and high)."""
    rng = random.Random(k)
    P = math.prod(modular.odd_primes_below(256))
    M = P ** k
    bits = M.bit_length() - 2
    for nb in (bits // 2, bits // 6, (5 * bits) // 6):
        db = bits - nb
        N, D = 1 << nb, 1 << db
        for _ in range(2):
            den = rng.randrange(1, D)
            num = rng.randrange(-N + 1, N)
            if math.gcd(den, M) != 1:
                continue
            a = num * pow(den, -1, M) % M
            assert ratrec(a, M, N, D) == dixon.rational_reconstruct(a, M, N, D)
    a = rng.randrange(M)
    half = bits // 2
    assert ratrec(a, M, 1 << half, 1 << half) == dixon.rational_reconstruct(a, M, 1 << half, 1 << half)


def test_ratrec_unbalanced_bounds_and_large_quotients():
    """Wang's stopping point away from the middle (N and D of different
    sizes), and remainder sequences with quotients of 2^62 and more (a full
    division) next to the one-word steps taken in place."""
    rng = random.Random(11)
    P = math.prod(modular.odd_primes_below(256))
    for k in [3, 20, 45]:
        M = P ** k
        bits = M.bit_length() - 2
        for nb in (bits // 5, bits // 2, (4 * bits) // 5):
            db = bits - nb
            N, D = 1 << nb, 1 << db
            for _ in range(6):
                den = rng.randrange(1, D)
                num = rng.randrange(-N + 1, N)
                if math.gcd(den, M) != 1:
                    continue
                a = num * pow(den, -1, M) % M
                assert ratrec(a, M, N, D) == dixon.rational_reconstruct(a, M, N, D)
            # quotients far above 2^62 early and late in the sequence
            for shift in (70, 200, nb // 2 + 64):
                a = M // (1 << shift) + rng.randrange(1 << 40)
                assert ratrec(a, M, N, D) == dixon.rational_reconstruct(a, M, N, D)
                small = rng.randrange(1, 1 << min(db - 1, 300))
                a = (small * ((1 << shift) + 1)) % M
                assert ratrec(a, M, N, D) == dixon.rational_reconstruct(a, M, N, D)


# ------------------------------------------------------------------ reconstruction stage

def digits_to_words(digits):
    """oracle digits [m][n][c] (Python ints) -> int64 [n*c][m][6] two's complement."""
    m, n, c = len(digits), len(digits[0]), len(digits[0][0])
    out = np.zeros((n * c, m, 6), dtype=np.uint64)
    for i in range(m):
        for r in range(n):
            for t in range(c):
                v = digits[i][r][t] % (1 << 384)
                for w in range(6):
                    out[r * c + t, i, w] = (v >> (64 * w)) & ((1 << 64) - 1)
    return out.view(np.int64)


def oracle_case(A, b, primes):
    live, invs = dixon.surviving_primes(A, primes)
    P = math.prod(live)
    N, D = dixon.hadamard_bounds(A, b)
    nbits, dbits = max(1, N.bit_length()), max(1, D.bit_length())
    m = dixon.step_count(P, 1 << nbits, 1 << dbits)
    digits, _ = dixon.padic_digits(A, b, live, m, B=dixon.crt_matrix(invs, live))
    mask = sum(1 << primes.index(q) for q in live)
    return digits_to_words(digits), mask, nbits, dbits


@pytest.mark.parametrize("case", ["c1_n32_int8", "c2_pascal30", "uniform", "hilbert", "planted", "zero_b",
                                  "int64_extremes"])
def test_reconstruct_matches_oracle(case, primes):
    if case.startswith("c"):
        A, b = W.generate(case)
    elif case == "uniform":
        A, b = W.uniform_system(24, 3, 24, 17)
    elif case == "hilbert":
        A, _ = W.scaled_hilbert(8)
        b = np.arange(16, dtype=np.int64).reshape(8, 2) - 7
    elif case == "planted":
        A, b, _ = W.planted_system(20, 2, 12, 16, 4)
    elif case == "zero_b":
        A, _ = W.uniform_system(9, 1, 16, 2)
        b = np.zeros((9, 2), dtype=np.int64)
    else:
        A = np.array([[3, (1 << 61)], [-(1 << 61), 5]], dtype=np.int64)
        b = np.array([[-(1 << 63)], [(1 << 63) - 1]], dtype=np.int64)
    n, c = A.shape[0], b.shape[1]
    words, mask, nbits, dbits = oracle_case(A, b, primes)
    got = es.reconstruct(words, n, c, mask, nbits, dbits, threads=3)
    assert got == exact.solve(A, b)


def test_reconstruct_rejects_short_precision(primes):
    A, b = W.uniform_system(6, 1, 16, 1)
    words, mask, nbits, dbits = oracle_case(A, b, primes)
    with pytest.raises(ValueError):
        es.reconstruct(words[:, :1], 6, 1, mask, nbits + 400, dbits + 400)


def test_step_count_without_forming_the_modulus():
    """The solve takes the lift's step count m (the least m with
    P^m > 2^(nbits + dbits + 1), card "Method") and the bit length of P^m from
    log2 P, forming P^m only while the GPU lifts.  It must agree with the
    exact powers, here also recomputed with Python integers, over random
    prime sets and bounds, including bounds that put k log2 P near an integer."""
    import random
    L = lib()
    f = L.es_dbg_step_count
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    primes = modular.odd_primes_below(256)
    rng = random.Random(5)
    me, be, mf, bf = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
    cases = []
    for _ in range(150):
        mask = rng.getrandbits(53) | 1
        cases.append((mask, rng.randrange(1, 40000), rng.randrange(1, 40000)))
    full = (1 << 53) - 1
    P = math.prod(primes)
    for k in (1, 2, 7, 50, 171, 172, 180):  # bounds that make P^k's bit length the exact threshold
        b = (P ** k).bit_length()
        cases += [(full, b - 2 - 1, 1), (full, b - 2, 1), (full, b - 2 + 1, 1)]
    for mask, nb, db in cases:
        if nb < 1:
            continue
        assert f(mask, nb, db, ctypes.byref(me), ctypes.byref(be), ctypes.byref(mf), ctypes.byref(bf)) == 0
        Pm = math.prod(q for j, q in enumerate(primes) if (mask >> j) & 1)
        need = nb + db + 2
        m = 1
        while (Pm ** m).bit_length() < need:
            m += 1
        assert (me.value, be.value) == (m, (Pm ** m).bit_length()), (mask, nb, db)
        assert (mf.value, bf.value) == (me.value, be.value), (mask, nb, db)
    assert f(0, 10, 10, ctypes.byref(me), ctypes.byref(be), ctypes.byref(mf), ctypes.byref(bf)) == -1
