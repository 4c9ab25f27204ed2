"""Complete exact check of A x == b for large solutions (test helper).

Used by the GPU parity tests at sizes where the Bareiss oracle is too slow to
run inline, and pinned on the CPU against the oracle (with planted errors) in
test_exact_check.py.  The solution of a nonsingular system is unique, so this
check together with lowest terms fixes every bit of the result.
"""
import math

import numpy as np


def _limbs16(v: int, nl: int):
    """|v| as nl little-endian 16-bit limbs (int64)."""
    return np.frombuffer(abs(v).to_bytes(2 * nl, "little"), dtype="<u2").astype(np.int64)


def exact_limb_check(A, b, X):
    """A x == b exactly, on every row and every column, for X given as
    [n][c] (num, den) pairs.

    Per column t, with L the lcm of the column's denominators and N = L x_t
    (integers), the integer vector V = A N - L b_t must vanish.  N, L and b
    are split into signed 16-bit limbs, so V_i = sum_k R[i, k] 2^(16 k) with
    integer limb sums R: the A N part is one float64 matrix product whose
    partial sums are integers below 2^53 in magnitude (asserted), hence
    exact; the L b part is a four-term limb convolution in int64.  Then
    V_i = 0 exactly when, carrying from the lowest limb up (c_0 = 0,
    v_k = R[i, k] + c_k), every v_k is a multiple of 2^16 and the final
    carry c_{k+1} = v_k / 2^16 is zero."""
    A = np.asarray(A, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    n, c = A.shape[0], b.shape[1]
    amax = int(np.abs(A).max())
    assert amax.bit_length() + 16 + n.bit_length() <= 53, "the float64 limb products would not be exact"
    Af = A.astype(np.float64)
    bs = np.sign(b).astype(np.int64)
    bl = np.stack([_limbs16(int(v), 4) for v in b.reshape(-1)]).reshape(n, c, 4)
    for t in range(c):
        L = 1
        for k in range(n):
            den = X[k][t][1]
            if L % den:
                L = L * den // math.gcd(L, den)
        N = [X[k][t][0] * (L // X[k][t][1]) for k in range(n)]
        bits = max(max(abs(v).bit_length() for v in N), L.bit_length() + 64)
        nl = (bits + amax.bit_length() + n.bit_length()) // 16 + 3
        Nl = np.stack([(-1 if v < 0 else 1) * _limbs16(v, nl) for v in N]).astype(np.float64)
        R = (Af @ Nl).astype(np.int64)                        # exact: |partial sums| < 2^53
        Ll = _limbs16(L, nl)
        for j in range(4):                                    # minus L b_t, limb by limb
            R[:, j:] -= (bs[:, t] * bl[:, t, j])[:, None] * Ll[None, :nl - j]
        carry = np.zeros(n, dtype=np.int64)
        for k in range(nl):
            v = R[:, k] + carry
            if np.any(v & 0xFFFF):
                return False
            carry = v >> 16
        if np.any(carry):
            return False
    return True
