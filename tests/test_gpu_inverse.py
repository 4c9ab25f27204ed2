"""GPU parity of the batched modular inverse (es_batched_inverse) against the oracle.

Element by element against the oracle's plain Gauss-Jordan mod q at sizes it
finishes in seconds (several row tiles, ragged tails, one and two column
passes), and by the defining identity B A = I (mod q) for every prime at the
full workload sizes.  Flags must equal "A singular mod q" as the oracle finds it.
"""
import numpy as np
import pytest
import torch

import dixon_adic_lifting_amd as es
from dixon_adic_lifting_amd import workloads as W
from oracle import modular

pytestmark = pytest.mark.gpu


def balanced_np(B, q):
    B = B % q
    return np.where(B > (q - 1) // 2, B - q, B).astype(np.int8)


def check_identity_gpu(A, B, flags, primes):
    """B_j A == I mod q_j for every live prime, exactly (fp64 products < 2^53)."""
    dev = B.device
    n = A.shape[0]
    At = torch.as_tensor(A, device=dev)
    eye = torch.eye(n, dtype=torch.float64, device=dev)
    for j, q in enumerate(primes):
        if flags[j]:
            continue
        Aq = torch.remainder(At, q).to(torch.float64)
        prod = torch.matmul(B[j].to(torch.float64), Aq)
        r = torch.remainder(prod, q)
        assert torch.equal(r, eye), f"B A != I mod {q}"


@pytest.mark.parametrize("n,bits,seed", [(1, 8, 1), (2, 8, 2), (5, 24, 3), (17, 24, 4), (32, 8, 5),
                                         (63, 24, 6), (64, 24, 7), (65, 16, 8), (100, 24, 9),
                                         (256, 24, 10)])
def test_inverse_elementwise(n, bits, seed, primes):
    A, _ = W.uniform_system(n, 1, bits, seed)
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    Bh = B.cpu().numpy()
    check_primes = primes if n <= 100 else primes[:3] + primes[-3:]
    for j, q in enumerate(primes):
        if q not in check_primes:
            continue
        ref = modular.inverse_mod(A, q)
        assert flags[j] == (1 if ref is None else 0), q
        if ref is not None:
            assert np.array_equal(Bh[j], balanced_np(ref, q)), q
    check_identity_gpu(A, B, flags, primes)


@pytest.mark.parametrize("n,seed", [(70, 11), (261, 12)])
def test_inverse_mixed_width_entries(n, seed, primes):
    """Entries below 2^24 mixed with entries of 33 to 54 bits in the same rows
    (and the same groups of four columns): each group is reduced from 64 bits
    when any of its entries needs them, from 32 bits otherwise."""
    A, _ = W.uniform_system(n, 1, 24, seed)
    rng = np.random.default_rng(seed)
    wide = rng.random((n, n)) < 0.1
    mags = rng.integers(1 << 32, 1 << 54, size=(n, n), dtype=np.int64)
    signs = rng.choice(np.array([-1, 1], dtype=np.int64), size=(n, n))
    A = np.where(wide, signs * mags, A)
    assert n * int(np.abs(A).max()) < (1 << 63)
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    Bh = B.cpu().numpy()
    for q in (primes[:3] + primes[-3:]):
        j = primes.index(q)
        ref = modular.inverse_mod(A, q)
        assert flags[j] == (1 if ref is None else 0), q
        if ref is not None:
            assert np.array_equal(Bh[j], balanced_np(ref, q)), q
    check_identity_gpu(A, B, flags, primes)


def test_inverse_pascal(primes):
    A, _ = W.generate("c2_pascal30")
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    assert flags == [0] * 53                      # unimodular: invertible mod every prime
    Bh = B.cpu().numpy()
    for j, q in enumerate(primes):
        assert np.array_equal(Bh[j], balanced_np(modular.inverse_mod(A, q), q))


def test_inverse_dropped_primes(primes):
    A, _ = W.uniform_system(40, 1, 12, 21)
    A[0] *= 3 * 7          # det divisible by 3 and 7
    A[1] *= 251
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    for j, q in enumerate(primes):
        ref = modular.inverse_mod(A, q)
        assert flags[j] == (1 if ref is None else 0)
        if ref is not None:
            assert np.array_equal(B[j].cpu().numpy(), balanced_np(ref, q))
    assert flags[primes.index(3)] == 1 and flags[primes.index(7)] == 1 and flags[primes.index(251)] == 1


def test_inverse_needs_pivoting(primes):
    # zero diagonal and a leading zero column block force non-trivial pivots
    rng = np.random.default_rng(4)
    n = 48
    A = rng.integers(-100, 100, size=(n, n), dtype=np.int64)
    for i in range(n):
        A[i, i] = 0
    A[: n // 2, 0] = 0
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    for j, q in enumerate(primes):
        ref = modular.inverse_mod(A, q)
        assert flags[j] == (1 if ref is None else 0)
        if ref is not None:
            assert np.array_equal(B[j].cpu().numpy(), balanced_np(ref, q))


def test_inverse_singular_everywhere():
    A, _ = W.duplicate_row_system(33, 2)
    _, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    assert flags == [1] * 53
    Z = np.zeros((20, 20), dtype=np.int64)
    _, flags = es.batched_inverse(torch.as_tensor(Z).cuda())
    assert flags == [1] * 53


def test_inverse_range_error():
    n = 4
    A = np.eye(n, dtype=np.int64)
    A[0, 0] = 1 << 61          # n * max = 2^63
    with pytest.raises(ValueError):
        es.batched_inverse(torch.as_tensor(A).cuda())
    A[0, 0] = (1 << 61) - 1    # n * max < 2^63: accepted
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    assert sum(flags) < 53


@pytest.mark.parametrize("name", ["c4_n1024_int24", "c5_n2048_c16_int24"])
def test_inverse_full_size(name, primes):
    A, _ = W.generate(name)
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    check_identity_gpu(A, B, flags, primes)
    # element-wise for the smallest and the largest prime (oracle GJ on the CPU)
    if A.shape[0] <= 1024:
        for q in (3, 251):
            j = primes.index(q)
            ref = modular.inverse_mod(A, q)
            assert flags[j] == (1 if ref is None else 0)
            if ref is not None:
                assert np.array_equal(B[j].cpu().numpy(), balanced_np(ref, q))


def test_inverse_ragged_two_passes(primes):
    # n > 1024 and not a multiple of 64: the second column pass is partly masked
    A, _ = W.uniform_system(1090, 1, 24, 31)
    B, flags = es.batched_inverse(torch.as_tensor(A).cuda())
    check_identity_gpu(A, B, flags, primes)


def both_inverses(A):
    """(B, flags) from the blocked elimination and from one launch per step.
    The blocked form runs twice: with each panel overlapping the previous
    panel's update (the default), and one kernel at a time (the form used
    while kernels are timed); the two must agree exactly."""
    from dixon_adic_lifting_amd import _lib
    dA = torch.as_tensor(A).cuda()
    try:
        _lib.set_blocked_inverse(True)
        Bb, fb = es.batched_inverse(dA)
        _lib.set_profiling(True)
        Bp, fp = es.batched_inverse(dA)
        _lib.set_profiling(False)
        assert fp == fb
        for j in range(53):
            if not fb[j]:
                assert torch.equal(Bb[j], Bp[j]), j
        _lib.set_blocked_inverse(False)
        Bs, fs = es.batched_inverse(dA)
    finally:
        _lib.set_profiling(False)
        _lib.set_blocked_inverse(True)
    return Bb, fb, Bs, fs


@pytest.mark.parametrize("n,bits,seed", [(1, 8, 31), (31, 24, 32), (32, 24, 33), (33, 8, 34), (97, 24, 35),
                                         (130, 4, 36), (300, 24, 37), (1090, 24, 38)])
def test_blocked_and_stepwise_inverse_agree(n, bits, seed, primes):
    # every prime's balanced inverse and every singular flag match bit for bit
    # (4-bit entries at n = 130 make several primes divide det A); n = 1090
    # has a ragged last panel and rows past one 1024-thread block
    A, _ = W.uniform_system(n, 1, bits, seed)
    Bb, fb, Bs, fs = both_inverses(A)
    assert fb == fs
    for j in range(53):
        if not fb[j]:
            assert torch.equal(Bb[j], Bs[j]), primes[j]


def test_blocked_inverse_pivoting_and_singular_primes(primes):
    # zero leading entries force pivots away from the diagonal; a rank-deficient
    # block makes every prime singular at a known step
    rng = np.random.default_rng(40)
    n = 70
    A = rng.integers(-50, 50, size=(n, n), dtype=np.int64)
    A[:40, :3] = 0
    Bb, fb, Bs, fs = both_inverses(A)
    assert fb == fs
    for j in range(53):
        if not fb[j]:
            assert torch.equal(Bb[j], Bs[j])
    check_identity_gpu(A, Bb, fb, primes)
    S = A.copy()
    S[:, 45] = S[:, 3] + 2 * S[:, 7]           # singular over Q: singular mod every prime
    Bb, fb, _, fs = both_inverses(S)
    assert fb == fs == [1] * 53
