"""Exact rational solution of integer systems A x = b on one MI355X.

Multi-prime Dixon p-adic lifting with hand-written HIP kernels for gfx950,
behind the C ABI in ``include/es_solve.h``; this package is a thin binding
(PyTorch supplies device memory and the current stream).  Method and limits
follow the exact-solve card (phanerozoic/exact-solve): ``solve(A, b)``
returns ``[n][c]`` exact ``fractions.Fraction`` values, or ``None`` when A is
singular over the rationals; ``A`` is ``[n, n]`` and ``b`` is ``[n, c]``,
integer, with ``n * max|A_ij| < 2^63`` and ``n <= 2^17``.
"""
from __future__ import annotations

import ctypes
from fractions import Fraction

import numpy as np

from . import _lib

__all__ = ["solve", "solve_pairs", "batched_inverse", "batched_inverse_noalloc", "noalloc_max_n", "lift_digits",
           "reconstruct", "primes", "workspace_bytes", "last_timings", "SolveError"]

NUM_PRIMES = _lib.NUM_PRIMES


class SolveError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"{_lib.strerror(status)} (status {status})")
        self.status = status


def _raise(status: int):
    if status in (_lib.ES_EINVAL, _lib.ES_ERANGE, _lib.ES_ETOOBIG):
        raise ValueError(f"{_lib.strerror(status)} (status {status})")
    raise SolveError(status)


def primes():
    buf = (ctypes.c_int32 * NUM_PRIMES)()
    _lib.load().es_primes(buf, NUM_PRIMES)
    return list(buf)


def workspace_bytes(n: int, c: int) -> int:
    return int(_lib.load().es_workspace_bytes(int(n), int(c)))


def last_timings():
    return _lib.last_timings()


def _device_inputs(A, b=None):
    import torch
    if not isinstance(A, torch.Tensor):
        A = torch.as_tensor(np.asarray(A))
    dev = A.device if A.is_cuda else torch.device("cuda", torch.cuda.current_device())
    if A.dim() != 2 or A.shape[0] != A.shape[1]:
        raise ValueError("A must be [n, n]")
    if A.dtype.is_floating_point or A.dtype.is_complex or A.dtype == torch.bool:
        raise ValueError("A must be an integer tensor")
    A = A.to(device=dev, dtype=torch.int64).contiguous()
    if b is None:
        return A, None, dev
    if not isinstance(b, torch.Tensor):
        b = torch.as_tensor(np.asarray(b))
    if b.dim() != 2 or b.shape[0] != A.shape[0]:
        raise ValueError("b must be [n, c]")
    if b.dtype.is_floating_point or b.dtype.is_complex or b.dtype == torch.bool:
        raise ValueError("b must be an integer tensor")
    b = b.to(device=dev, dtype=torch.int64).contiguous()
    return A, b, dev


def _workspace(n: int, c: int, dev):
    import torch
    nbytes = workspace_bytes(n, c)
    if nbytes == 0:
        raise ValueError("n or c out of range")
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def solve_pairs(A, b, workspace=None):
    """x = A^-1 b as [n][c] (num, den) integer pairs in lowest terms, or None if singular."""
    lib = _lib.load()
    A, b, dev = _device_inputs(A, b)
    n, c = A.shape[0], b.shape[1]
    ws = workspace if workspace is not None else _workspace(n, c, dev)
    sol = ctypes.c_void_p()
    st = lib.es_solve_device(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, c,
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev), ctypes.byref(sol))
    if st == _lib.ES_SINGULAR:
        return None
    if st != _lib.ES_OK:
        _raise(st)
    try:
        return _lib.read_solution(sol)
    finally:
        lib.es_solution_free(sol)


def solve(A, b, workspace=None):
    """Exact solution: ``[n][c]`` nested lists of ``Fraction``; ``None`` if A is singular."""
    pairs = solve_pairs(A, b, workspace)
    if pairs is None:
        return None
    return [[Fraction(p, q) for (p, q) in row] for row in pairs]


def solve_info(A, b, workspace=None):
    """(pairs or None, info dict with live_primes, m, bound bits, stage timings)."""
    lib = _lib.load()
    A, b, dev = _device_inputs(A, b)
    n, c = A.shape[0], b.shape[1]
    ws = workspace if workspace is not None else _workspace(n, c, dev)
    sol = ctypes.c_void_p()
    st = lib.es_solve_device(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, c,
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev), ctypes.byref(sol))
    if st == _lib.ES_SINGULAR:
        return None, {"status": st, **last_timings()}
    if st != _lib.ES_OK:
        _raise(st)
    try:
        return _lib.read_solution(sol), {"status": st, **_lib.solution_info(sol), **last_timings()}
    finally:
        lib.es_solution_free(sol)


def batched_inverse(A, workspace=None):
    """(B, flags): B int8 [53][n][n] device tensor of balanced A^-1 mod q_j; flags[j] = 1 if singular mod q_j."""
    import torch
    lib = _lib.load()
    A, _, dev = _device_inputs(A)
    n = A.shape[0]
    ws = workspace if workspace is not None else _workspace(n, 1, dev)
    B = torch.empty((NUM_PRIMES, n, n), dtype=torch.int8, device=dev)
    flags = (ctypes.c_int32 * NUM_PRIMES)()
    st = lib.es_batched_inverse(ctypes.c_void_p(A.data_ptr()), n, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                _stream(dev), ctypes.c_void_p(B.data_ptr()), flags)
    if st != _lib.ES_OK:
        _raise(st)
    return B, list(flags)


def batched_inverse_noalloc(A, out=None):
    """The same as ``batched_inverse`` through the entry point that allocates
    nothing on the device (fixed scratch, n <= noalloc_max_n()).  ``out`` may
    supply the int8 [53][n][n] result tensor."""
    import torch
    lib = _lib.load()
    A, _, dev = _device_inputs(A)
    n = A.shape[0]
    B = out if out is not None else torch.empty((NUM_PRIMES, n, n), dtype=torch.int8, device=dev)
    if B.dtype != torch.int8 or tuple(B.shape) != (NUM_PRIMES, n, n) or not B.is_contiguous():
        raise ValueError("out must be a contiguous int8 [53][n][n] tensor")
    flags = (ctypes.c_int32 * NUM_PRIMES)()
    st = lib.es_batched_inverse_noalloc(ctypes.c_void_p(A.data_ptr()), n, _stream(dev), ctypes.c_void_p(B.data_ptr()),
                                        flags)
    if st != _lib.ES_OK:
        _raise(st)
    return B, list(flags)


def noalloc_max_n() -> int:
    return int(_lib.load().es_noalloc_max_n())


def lift_digits(A, b, m: int = 0, workspace=None):
    """(digits int64 [n*c][m][6], live_mask, m) -- the lift's base-P digits, 384-bit two's complement.

    With m = 0 the step count comes from the Hadamard bound (one extra call
    sizes the buffer).  Returns None if A is singular.
    """
    lib = _lib.load()
    A, b, dev = _device_inputs(A, b)
    n, c = A.shape[0], b.shape[1]
    ws = workspace if workspace is not None else _workspace(n, c, dev)
    mask = ctypes.c_uint64()
    mout = ctypes.c_int32()
    args = (ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, c,
            ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev), int(m))
    if m <= 0:
        st = lib.es_lift_digits(*args, None, 0, ctypes.byref(mask), ctypes.byref(mout))
        if st == _lib.ES_SINGULAR:
            return None
        if st != _lib.ES_OK:
            _raise(st)
        m = mout.value
        args = args[:-1] + (m,)
    digits = np.zeros(n * c * m * _lib.DIGIT_LIMBS, dtype=np.int64)
    st = lib.es_lift_digits(*args, digits.ctypes.data_as(_lib.c_i64p), digits.size, ctypes.byref(mask),
                            ctypes.byref(mout))
    if st == _lib.ES_SINGULAR:
        return None
    if st != _lib.ES_OK:
        _raise(st)
    return digits.reshape(n * c, m, _lib.DIGIT_LIMBS), mask.value, m


def reconstruct(digits, n: int, c: int, live_mask: int, num_bits: int, den_bits: int, threads: int = 0):
    """Host rational reconstruction from digits [n*c][m][6]: [n][c] (num, den) pairs."""
    lib = _lib.load()
    d = np.ascontiguousarray(digits, dtype=np.int64)
    m = d.shape[1]
    sol = ctypes.c_void_p()
    st = lib.es_reconstruct(d.ctypes.data_as(_lib.c_i64p), n, c, m, int(live_mask), int(num_bits),
                            int(den_bits), int(threads), ctypes.byref(sol))
    if st != _lib.ES_OK:
        _raise(st)
    try:
        return _lib.read_solution(sol)
    finally:
        lib.es_solution_free(sol)
