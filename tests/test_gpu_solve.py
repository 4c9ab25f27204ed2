"""End-to-end GPU parity of es_solve_device against the oracle.

Bit-exact (numerators and denominators as integers) against the Bareiss
oracle on the small configurations, against the oracle's stored digests
(tests/golden/oracle_digests.json, written by tests/golden/make_golden.py,
which calls only oracle/) where the oracle is too slow to run inline, and at
every size by the properties that determine the answer uniquely: lowest
terms, positive denominators, and A x == b in exact integer arithmetic.
"""
import hashlib
import json
import math
import os

import numpy as np
import pytest
import torch

import dixon_adic_lifting_amd as es
from dixon_adic_lifting_amd import _lib, workloads as W
from oracle import cbareiss, exact, modular

from exact_check import exact_limb_check

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_digests.json")


def digest(X):
    def h(v):
        return ("-" + format(-v, "x")) if v < 0 else format(v, "x")
    return hashlib.sha256("".join(f"{h(p)} {h(q)}\n" for row in X for (p, q) in row).encode()).hexdigest()


def golden(name):
    with open(GOLDEN) as f:
        return json.load(f).get(name)


def solve_gpu(A, b):
    return es.solve_pairs(torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda())


def assert_normal_form(X):
    for row in X:
        for (p, q) in row:
            assert q > 0 and math.gcd(p, q) == 1 and (p != 0 or q == 1)


@pytest.mark.parametrize("name", ["c1_n32_int8", "c2_pascal30"])
def test_solve_small_configs_bit_exact(name):
    A, b = W.generate(name)
    X = solve_gpu(A, b)
    assert X == exact.solve(A, b)
    g = golden(name)
    assert g is not None and digest(X) == g["sha256"]
    if name == "c2_pascal30":
        assert all(q == 1 for row in X for (_, q) in row)     # unimodular -> integral


def test_solve_c3_bit_exact():
    A, b = W.generate("c3_n256_int24")
    X = solve_gpu(A, b)
    assert digest(X) == golden("c3_n256_int24")["sha256"]
    assert_normal_form(X)
    assert exact.check_solution(A, b, X)


def test_solve_c4():
    A, b = W.generate("c4_n1024_int24")
    X = solve_gpu(A, b)
    assert_normal_form(X)
    assert exact.check_solution(A, b, X)      # unique solution: this pins every bit
    g = golden("c4_n1024_int24")
    if g is not None:
        assert digest(X) == g["sha256"]


MOD_PRIMES = [1048573, 1048571, 1048559, 1048549, 1048517]   # primes below 2^20


def check_mod_primes(A, b, X, rows, primes=MOD_PRIMES):
    """A x == b modulo several 20-bit primes (int64 products stay exact),
    plus exact integer checks of A x == b on sampled rows."""
    n, c = A.shape[0], b.shape[1]
    for p in primes:
        xm = np.array([[(num % p) * pow(den % p, -1, p) % p for (num, den) in row] for row in X], dtype=np.int64)
        lhs = (np.mod(A, p).astype(np.int64) @ xm) % p
        assert np.array_equal(lhs, np.mod(b, p)), p
    for t in range(c):
        L = 1
        for k in range(n):
            if L % X[k][t][1]:
                L = L * X[k][t][1] // math.gcd(L, X[k][t][1])
        col = [X[k][t][0] * (L // X[k][t][1]) for k in range(n)]
        for r in rows:
            assert sum(int(A[r, k]) * col[k] for k in range(n)) == L * int(b[r, t]), (r, t)


def test_solve_c5():
    """n = 2048, c = 16: complete exact check (every row and column) and
    lowest terms; the solve allocates no device memory beyond the inputs and
    the workspace it is handed."""
    A, b = W.generate("c5_n2048_c16_int24")
    dA, db = torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda()
    ws = torch.empty(es.workspace_bytes(2048, 16), dtype=torch.uint8, device="cuda")
    solve_gpu(A[:64, :64].copy(), b[:64].copy())        # the library's code objects are loaded
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    X = es.solve_pairs(dA, db, workspace=ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free0 - free1 < (2 << 20), (free0, free1)
    assert len(X) == 2048 and len(X[0]) == 16
    # every numerator came out of the GPU pass (a wrong product would push
    # components outside the bound and onto the host)
    alone, _ = _lib.last_recon_counts()
    assert alone == 0, alone
    assert_normal_form(X)
    assert exact_limb_check(A, b, X)


@pytest.mark.parametrize("n,c", [(128, 1), (512, 1), (256, 16), (512, 16)])
def test_card_table_shapes(n, c):
    """The card's other measured shapes (24-bit entries), drawn as the bench
    sweep draws them, checked completely: lowest terms and A x = b exactly
    on every row and column (the solution is unique, so this fixes every
    bit)."""
    A, b = W.uniform_system(n, c, 24, 1000 + n + c)
    X = solve_gpu(A, b)
    assert len(X) == n and len(X[0]) == c
    assert_normal_form(X)
    assert exact_limb_check(A, b, X)


# ------------------------------------------------------------------ edge families

def test_n1():
    for a, bb in [(7, 3), (-5, 10), (1, -(1 << 63)), ((1 << 62), 1)]:
        A = np.array([[a]], dtype=np.int64)
        b = np.array([[bb]], dtype=np.int64)
        assert solve_gpu(A, b) == exact.solve(A, b)


def test_zero_rhs_and_identity():
    A, _ = W.uniform_system(50, 1, 24, 3)
    b = np.zeros((50, 2), dtype=np.int64)
    assert solve_gpu(A, b) == [[(0, 1), (0, 1)] for _ in range(50)]
    I = np.eye(40, dtype=np.int64)
    b = np.arange(-40, 40, dtype=np.int64).reshape(40, 2)
    assert solve_gpu(I, b) == [[(int(v), 1) for v in row] for row in b]


def test_int64_extremes_in_b():
    A, b = W.uniform_system(20, 3, 24, 4)
    b[0, 0] = np.iinfo(np.int64).min
    b[5, 2] = np.iinfo(np.int64).max
    b[7, 1] = np.iinfo(np.int64).min + 1
    assert solve_gpu(A, b) == exact.solve(A, b)


def test_range_limit_edges():
    n = 8
    rng = np.random.default_rng(5)
    A = rng.integers(-1000, 1000, size=(n, n), dtype=np.int64)
    b = rng.integers(-1000, 1000, size=(n, 1), dtype=np.int64)
    A[2, 3] = ((1 << 63) - 1) // n            # n * max <= 2^63 - 1: accepted
    assert solve_gpu(A, b) == exact.solve(A, b)
    A[2, 3] = (1 << 63) // n                  # n * max = 2^63: rejected
    with pytest.raises(ValueError):
        solve_gpu(A, b)
    A[2, 3] = np.iinfo(np.int64).min          # |INT64_MIN| handled without overflow
    with pytest.raises(ValueError):
        solve_gpu(A, b)


def test_dropped_prime_path():
    A, b = W.uniform_system(30, 2, 20, 6)
    A[0] *= 3
    A[3] *= 11 * 251
    X, info = es.solve_info(torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda())
    assert info["live_primes"] <= 50
    assert X == exact.solve(A, b)


@pytest.mark.parametrize("maker", ["dup", "zero_col", "zero_row", "low_rank", "big_dup"])
def test_singular_families(maker):
    if maker == "dup":
        A, b = W.duplicate_row_system(12, 1)
    elif maker == "zero_col":
        A, b = W.zero_column_system(12, 2)
    elif maker == "zero_row":
        A, b = W.uniform_system(12, 1, 16, 3)
        A[4] = 0
    elif maker == "low_rank":
        A, b = W.low_rank_system(16, 9, 3)
    else:   # int24 entries at n = 256: the bound exceeds prod(q), so the rank test decides
        A, b = W.uniform_system(256, 1, 24, 11)
        A[200] = A[10]
    assert solve_gpu(A, b) is None


def test_nonsingular_but_every_prime_divides_det():
    qs = modular.odd_primes_below(256)
    A = np.diag(qs).astype(np.int64)
    b = np.arange(1, 54, dtype=np.int64).reshape(53, 1)
    with pytest.raises(es.SolveError) as ei:
        solve_gpu(A, b)
    assert ei.value.status == -3


def test_scaled_hilbert_dense_denominators():
    for n in (6, 12, 21):
        A, L = W.scaled_hilbert(n)
        assert n * L < (1 << 63)
        b = np.arange(2 * n, dtype=np.int64).reshape(n, 2) - n
        X = solve_gpu(A, b)
        assert X == exact.solve(A, b)
        assert any(q > 1 for row in X for (_, q) in row)


def test_planted_integer_solution():
    A, b, Xs = W.planted_system(128, 3, 20, 20, 9)
    assert solve_gpu(A, b) == [[(int(v), 1) for v in row] for row in Xs]


@pytest.mark.parametrize("n,c,bits,seed", [(33, 17, 24, 1), (100, 5, 30, 2), (129, 1, 24, 3),
                                           (300, 2, 16, 4), (64, 16, 40, 5), (40, 3, 32, 7)])
def test_random_shapes_vs_c_oracle(n, c, bits, seed):
    A, b = W.uniform_system(n, c, bits, seed)
    X = solve_gpu(A, b)
    assert X == cbareiss.solve(A, b)


def test_ragged_two_pass_width():
    A, b = W.uniform_system(1090, 1, 24, 12)
    X = solve_gpu(A, b)
    assert_normal_form(X)
    check_mod_primes(A, b, X, rows=[0, 1089])


def test_deterministic_bytes():
    A, b = W.uniform_system(200, 3, 24, 13)
    X1 = solve_gpu(A, b)
    X2 = solve_gpu(A, b)
    assert X1 == X2 and digest(X1) == digest(X2)


def test_host_pointer_entry_matches_device_entry():
    import ctypes
    from dixon_adic_lifting_amd import _lib
    A, b = W.generate("c1_n32_int8")
    lib = _lib.load()
    sol = ctypes.c_void_p()
    Ac = np.ascontiguousarray(A)
    bc = np.ascontiguousarray(b)
    st = lib.es_solve(Ac.ctypes.data_as(_lib.c_i64p), bc.ctypes.data_as(_lib.c_i64p), 32, 1, ctypes.byref(sol))
    assert st == 0
    try:
        assert _lib.read_solution(sol) == solve_gpu(A, b)
    finally:
        lib.es_solution_free(sol)


def test_bad_arguments():
    A = torch.zeros((4, 4), dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        es.solve_pairs(A, torch.zeros(4, dtype=torch.int64, device="cuda"))          # 1-D b
    with pytest.raises(ValueError):
        es.solve_pairs(torch.zeros((4, 5), dtype=torch.int64, device="cuda"), torch.zeros((4, 1), dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        es.solve_pairs(A.double(), torch.zeros((4, 1), dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("c", [1, 2])
def test_first_samples_miss_a_factor_of_the_denominator(c):
    """With one right-hand side the GPU reconstruction starts its pass from
    the lcm of the first two sample components' denominators and checks it
    against the whole sample's lcm (card, "Method": d is the lcm over the
    sample); with several it waits for the whole sample.  Here every column
    of x is u + v / 7 with v zero in rows 0 and 2 (for n = 16 the first two
    samples are components 0 and 2 at c = 1), so those are integers while
    other components have denominator 7: at c = 1 the first pass is dropped
    and run again with the whole sample's d; at c = 2 the whole sample gives
    d at once.  Either way the result must be exact."""
    n = 16
    rng = np.random.default_rng(31)
    A = rng.integers(-50, 50, size=(n, n), dtype=np.int64)
    U = rng.integers(-1000, 1000, size=(n, c), dtype=np.int64)
    V = rng.integers(1, 7, size=(n, c), dtype=np.int64)
    V[0, :] = V[2, :] = 0
    # column 5 of A makes A V = 0 (mod 7) for the first column of V ...
    k = 5
    v = V[:, 0]
    rest = (A @ v - A[:, k] * v[k]) % 7
    A[:, k] = (-(rest * pow(int(v[k]), -1, 7)) % 7) + 7 * rng.integers(-5, 5, size=n)
    # ... and the other columns of V are multiples of it mod 7
    for t in range(1, c):
        V[:, t] = (V[:, 0] * (t + 1)) % 7
    assert np.all((A @ V) % 7 == 0)
    b = A @ U + (A @ V) // 7
    got = solve_gpu(A, b)
    ref = exact.solve(A, b)
    assert got == ref
    for t in range(c):
        assert ref[0][t][1] == 1 and ref[2][t][1] == 1
        assert math.lcm(*(row[t][1] for row in ref)) % 7 == 0


def test_mfma_residual_plane_extremes():
    """Several right-hand sides with |A| < 2^30 take the residual as int8 MFMA
    products of A's four balanced byte planes and x's eight; entries at
    +-(2^30 - 1), +-2^23 and -1, 0, 1 exercise every plane's extremes (the
    top plane of 2^30 - 1 is 64, of -(2^30 - 1) is -64)."""
    n, c = 24, 3
    A, b = W.uniform_system(n, c, 24, 17)
    A[0, 0] = (1 << 30) - 1
    A[1, 5] = -((1 << 30) - 1)
    A[2, 7] = 1 << 23
    A[3, 9] = -(1 << 23)
    A[4, 4], A[5, 5], A[6, 6] = -1, 0, 1
    X = solve_gpu(A, b)
    assert X == cbareiss.solve(A, b)


def test_modulus_with_a_full_top_word():
    """A modulus M = P^m whose bit length is a multiple of 32 (its top 32-bit
    word at least 2^31).  The GPU reconstruction keeps weights and numerators
    in [0, 2M), one bit above M, so its word window must reach past M's top
    word; otherwise every numerator leaves the bound and falls back to the
    host.  With all 53 primes live, m = 23 gives such a modulus; 64 x 64
    systems with 50-56-bit entries land near it."""
    hit = None
    for bits in range(50, 57):
        for seed in range(12):
            A, b = W.uniform_system(64, 1, bits, 7000 + 100 * bits + seed)
            X, info = es.solve_info(torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda())
            if X is not None and info["modulus_bits"] % 32 == 0:
                hit = (A, b, X)
                break
        if hit:
            break
    assert hit is not None, "no 32-aligned modulus among the draws"
    A, b, X = hit
    alone, host_gcds = _lib.last_recon_counts()
    assert alone == 0 and host_gcds >= 0, (alone, host_gcds)
    assert_normal_form(X)
    assert exact.check_solution(A, b, X)
