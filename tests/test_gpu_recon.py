"""GPU reconstruction (one int8 MFMA GEMM for every component's modular
multiply y = d X mods M) against the host reconstruction and the oracle.

* the GPU path and the host path return identical fractions on the same
  digits, for random shapes (including a ragged chunk of components and
  several right-hand sides) and at the n = 256 configuration;
* components whose denominator the sample misses (|y| > N) fall back to
  reconstruction on their own and still match the oracle;
* numerators of both signs, zero numerators and b = 0;
* the result of the GPU path against the Bareiss oracle on small systems.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import dixon_adic_lifting_amd as es
from dixon_adic_lifting_amd import _lib
from dixon_adic_lifting_amd import workloads as W
from oracle import exact

pytestmark = pytest.mark.gpu


def solve_both(A, b):
    dA, db = torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda()
    try:
        _lib.set_gpu_reconstruction(True)
        Xg = es.solve_pairs(dA, db)
        _lib.set_gpu_reconstruction(False)
        Xh = es.solve_pairs(dA, db)
    finally:
        _lib.set_gpu_reconstruction(True)
    return Xg, Xh


@pytest.mark.parametrize("n,c,bits,seed", [(1, 1, 24, 11), (5, 3, 8, 12), (40, 1, 24, 13), (97, 2, 16, 14),
                                           (130, 5, 24, 15), (300, 1, 24, 16)])
def test_gpu_and_host_reconstruction_agree(n, c, bits, seed):
    A, b = W.uniform_system(n, c, bits, seed)
    Xg, Xh = solve_both(A, b)
    assert Xg == Xh
    if n <= 40:
        assert Xg == exact.solve(A, b)


def test_gpu_reconstruction_c3():
    A, b = W.generate("c3_n256_int24")
    Xg, Xh = solve_both(A, b)
    assert Xg == Xh
    assert exact.check_solution(A, b, Xg)


def test_components_the_sample_misses():
    # x_i = b_i / (i + 1): the sample (components 0, 4, 8, 12) gives
    # d = lcm(1, 5, 9, 13), so most components exceed the numerator bound
    # after the modular multiply and are reconstructed alone
    n = 16
    A = np.diag(np.arange(1, n + 1)).astype(np.int64)
    rng = np.random.default_rng(21)
    b = rng.integers(-1000, 1000, size=(n, 1), dtype=np.int64)
    Xg, Xh = solve_both(A, b)
    want = [[(Fraction(int(b[i, 0]), i + 1).numerator, Fraction(int(b[i, 0]), i + 1).denominator)]
            for i in range(n)]
    assert Xg == want and Xh == want


def test_signs_and_zero_numerators():
    rng = np.random.default_rng(22)
    n = 24
    A = rng.integers(-50, 50, size=(n, n), dtype=np.int64)
    A += np.eye(n, dtype=np.int64) * 200
    x = rng.integers(-9, 9, size=(n, 2), dtype=np.int64)
    x[::3, 0] = 0
    b = A @ x                                 # planted integer solution, zeros and both signs
    Xg, Xh = solve_both(A, b)
    assert Xg == Xh == [[(int(x[i, t]), 1) for t in range(2)] for i in range(n)]
    b0 = np.zeros((n, 1), dtype=np.int64)
    Xg, _ = solve_both(A, b0)
    assert Xg == [[(0, 1)] for _ in range(n)]


@pytest.mark.parametrize("n,c,seed", [(257, 1, 31), (267, 3, 34), (301, 4, 32), (521, 8, 33)])
def test_gcd_groups_and_partial_blocks(n, c, seed):
    """The gcd kernel runs several components per block (one limb wave each;
    a Euclid wave for two of them on wide windows, four matrices a round,
    in blocks of up to four, else for eight of them on narrow windows), as
    many as the component count spread over the compute units asks for, up
    to thirteen, and three or four per compute unit as two blocks of two.
    n c = 257, 801, 1204 and 4168 components give groups of 2, 2, 5 and 13
    (256 compute units): both window forms, each with a partial last block
    (a lone component in the first case); the GPU path must match the host path and
    reconstruct no component alone.  A gcd goes back to the host only when a Euclidean quotient
    reaches 2^26 (about 2e-8 per step by the Gauss-Kuzmin law, so about once
    in the 3e7 steps of the largest case) or the gcd exceeds 64 bits."""
    A, b = W.uniform_system(n, c, 24, seed)
    dA, db = torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda()
    Xg = es.solve_pairs(dA, db)
    alone, host_gcds = _lib.last_recon_counts()
    assert alone == 0 and 0 <= host_gcds <= 3, (alone, host_gcds)
    try:
        _lib.set_gpu_reconstruction(False)
        Xh = es.solve_pairs(dA, db)
    finally:
        _lib.set_gpu_reconstruction(True)
    assert Xg == Xh
    assert any(q != max(qq for row in Xg for (_, qq) in row) for row in Xg for (_, q) in row) or n * c < 300


@pytest.mark.gpu
def test_gcds_in_two_launches():
    """With many components the gcd blocks take several rounds of the
    compute units, and the gcds go as two launches (the host finishes the
    first launch's components while the second runs).  n = 48 and c = 640
    give 30720 short components: 2364 blocks of thirteen, five rounds of two
    blocks per compute unit, split four rounds to one.  The result must
    match the host path, with no component reconstructed alone."""
    n, c = 48, 640
    A, b = W.uniform_system(n, c, 24, 41)
    dA, db = torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda()
    try:
        _lib.set_profiling(True)
        Xg = es.solve_pairs(dA, db)
        prof = _lib.kernel_profile()
    finally:
        _lib.set_profiling(False)
    alone, host_gcds = _lib.last_recon_counts()
    assert alone == 0 and 0 <= host_gcds <= 3, (alone, host_gcds)
    assert prof["recon_gcd"][1] == 2, prof["recon_gcd"]
    try:
        _lib.set_gpu_reconstruction(False)
        Xh = es.solve_pairs(dA, db)
    finally:
        _lib.set_gpu_reconstruction(True)
    assert Xg == Xh


@pytest.mark.gpu
def test_large_numerator_product_tiles():
    """n = 1024, c = 8: 8192 components against weight rows of about 6900
    bytes, enough 256 x 256 tiles to give every compute unit two blocks, so
    the numerators come from the large-tile product kernel.  Every component
    must be accepted on the GPU (a wrong product sends components outside
    the bound) and match the host path."""
    A, b = W.uniform_system(1024, 8, 24, 43)
    dA, db = torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda()
    Xg = es.solve_pairs(dA, db)
    alone, host_gcds = _lib.last_recon_counts()
    assert alone == 0 and 0 <= host_gcds <= 3, (alone, host_gcds)
    try:
        _lib.set_gpu_reconstruction(False)
        Xh = es.solve_pairs(dA, db)
    finally:
        _lib.set_gpu_reconstruction(True)
    assert Xg == Xh


def _sample_rule(NC, c):
    # the reconstruction's sample: the first row, then the k-th of seven
    # more components at k NC / 8 + (k mod c)
    s = list(range(min(c, NC)))
    for k in range(1, 8):
        j = k * NC // 8 + k % c
        if c <= j < NC and j not in s:
            s.append(j)
    return s


@pytest.mark.gpu
def test_several_rhs_sample_missing_a_factor_two():
    """n = 40, c = 16, seed 5029: the sample's denominators have an lcm that
    lacks a factor 2 which 128 of the 640 components' denominators carry (a
    pattern that random systems with sixteen right-hand sides show about
    one time in twenty).  The pass's d carries 2^2 beyond the sample's lcm,
    so every component is accepted in the one pass (none outside the bound)
    and the result is the oracle's."""
    n, c = 40, 16
    A, b = W.uniform_system(n, c, 24, 5029)
    ref = exact.solve(A, b)
    dens = [d for row in ref for (_, d) in row]
    ds = 1
    for j in _sample_rule(n * c, c):
        ds = ds * dens[j] // math.gcd(ds, dens[j])
    assert sum(1 for d in dens if ds % d) == 128     # the case: the sample misses a factor
    X = es.solve_pairs(torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda())
    alone, _ = _lib.last_recon_counts()
    assert alone == 0, alone
    assert X == ref


@pytest.mark.parametrize("diag,c", [((8388593, 8388587), 1), ((8388593, 8388587, 8388581, 8388571, 8388547), 1),
                                    ((8388593, 8388587, 8388581), 3)])
def test_tight_denominator_bound(diag, c):
    """Diagonal systems whose entries are distinct primes near 2^23: the
    common denominator is the whole determinant, which equals the Hadamard
    bound, so the small factors the pass's d takes beyond the sample's lcm
    do not fit under the denominator bound (d stays the lcm) and the
    numerators d x reach the numerator bound.  The result must still be
    the oracle's, in lowest terms."""
    n = len(diag)
    A = np.diag(np.array(diag, dtype=np.int64))
    rng = np.random.default_rng(n + c)
    b = rng.integers(-(1 << 22), 1 << 22, size=(n, c), dtype=np.int64)
    X = es.solve_pairs(torch.as_tensor(A).cuda(), torch.as_tensor(b).cuda())
    assert X == exact.solve(A, b)
