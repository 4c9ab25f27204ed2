"""ctypes loader for the plain-C Bareiss oracle (oracle/bareiss.c).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  ``build()`` compiles the C
source with gcc into ``oracle/liboracle_bareiss.so``; ``solve`` runs it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "bareiss.c")
LIB = os.path.join(_HERE, "liboracle_bareiss.so")
_lib = None


def build() -> str:
    """Compile the C oracle (gcc, -O2, POSIX threads) in place."""
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-shared", "-fPIC", "-pthread",
                           "-Wall", "-Wno-unused-function", SRC, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        lib.oracle_solve.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_char_p)]
        lib.oracle_solve.restype = ctypes.c_int
        lib.oracle_solve_timed.argtypes = lib.oracle_solve.argtypes + [ctypes.POINTER(ctypes.c_double)]
        lib.oracle_solve_timed.restype = ctypes.c_int
        lib.oracle_free.argtypes = [ctypes.c_char_p]
        lib.oracle_free.restype = None
        lib.oracle_entry_update_seconds.argtypes = [ctypes.c_int] * 4
        lib.oracle_entry_update_seconds.restype = ctypes.c_double
        u64p = ctypes.POINTER(ctypes.c_uint64)
        for fn in (lib.oracle_dbg_divexact, lib.oracle_dbg_gcd):
            fn.argtypes = [u64p, ctypes.c_int, u64p, ctypes.c_int, u64p, ctypes.POINTER(ctypes.c_int),
                           ctypes.c_int]
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def run(A, b, threads: int | None = None, max_steps: int = -1, step_seconds=None):
    """Raw call: returns (status, text or None).  status 0 ok, 1 singular, 2 stopped.

    step_seconds: optional float64 numpy array of length n that receives the
    wall time of each elimination step.
    """
    lib = _load()
    A = np.ascontiguousarray(A, dtype=np.int64)
    b = np.ascontiguousarray(b, dtype=np.int64)
    n = A.shape[0]
    c = b.shape[1]
    assert A.shape == (n, n) and b.shape == (n, c)
    out = ctypes.c_char_p()
    args = (A.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            n, c, int(threads or default_threads()), int(max_steps), ctypes.byref(out))
    if step_seconds is not None:
        assert step_seconds.dtype == np.float64 and step_seconds.size >= n
        st = lib.oracle_solve_timed(*args, step_seconds.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    else:
        st = lib.oracle_solve(*args)
    if st < 0:
        raise ValueError("oracle_solve rejected its arguments")
    text = None
    if out.value is not None:
        text = out.value.decode()
        lib.oracle_free(out)
    return st, text


def solve(A, b, threads: int | None = None):
    """x = A^-1 b as [n][c] (num, den) pairs in lowest terms, or None if singular."""
    st, text = run(A, b, threads)
    if st == 1:
        return None
    assert st == 0
    n, c = np.asarray(A).shape[0], np.asarray(b).shape[1]
    vals = [tuple(int(tok, 16) for tok in line.split()) for line in text.splitlines()]
    assert len(vals) == n * c
    return [vals[r * c:(r + 1) * c] for r in range(n)]


def _limbs(v: int):
    v = abs(v)
    out = []
    while v:
        out.append(v & (2**64 - 1))
        v >>= 64
    return (ctypes.c_uint64 * max(1, len(out)))(*out), len(out)


def _bignum_call(fn, a: int, b: int):
    lib = _load()
    A, la = _limbs(a)
    B, lb = _limbs(b)
    cap = max(la, lb) + 2
    R = (ctypes.c_uint64 * cap)()
    lr = ctypes.c_int(0)
    st = getattr(lib, fn)(A, la, B, lb, R, ctypes.byref(lr), cap)
    return st, sum(int(R[i]) << (64 * i) for i in range(lr.value))


def divexact_magnitudes(a: int, b: int):
    """|a| / |b| by the C oracle's exact division, or None if it reports that
    |b| does not divide |a| (test hook)."""
    st, q = _bignum_call("oracle_dbg_divexact", a, b)
    if st == 1:
        return None
    assert st == 0
    return q


def gcd_magnitudes(a: int, b: int) -> int:
    """gcd(|a|, |b|) by the C oracle's binary gcd (test hook)."""
    st, g = _bignum_call("oracle_dbg_gcd", a, b)
    assert st == 0
    return g


def entry_update_seconds(limbs: int, prev_limbs: int, reps: int, threads: int) -> float:
    """Mean wall time of one elimination entry update (two products of
    `limbs`-limb numbers, their difference, the exact division by a
    `prev_limbs`-limb number) with `threads` threads running at once
    (measurement hook for the CPU baseline)."""
    v = _load().oracle_entry_update_seconds(int(limbs), int(prev_limbs), int(reps), int(threads))
    if v < 0:
        raise ValueError("bad arguments")
    return v
