"""ctypes binding to ``libexact_solve.so`` (argument marshalling only).

Every step of the solve runs in the HIP library; this module only turns
torch tensors into device pointers and the current HIP stream, and turns the
library's limbs into Python integers.  It raises if the library has not been
built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexact_solve.so")

ES_OK, ES_SINGULAR = 0, 1
ES_EINVAL, ES_ERANGE, ES_ENOPRIME, ES_EHIP, ES_ENOMEM, ES_EINTERNAL, ES_ETOOBIG = -1, -2, -3, -4, -5, -6, -7
NUM_PRIMES = 53
DIGIT_LIMBS = 6

EXPORTS = ["es_strerror", "es_primes", "es_workspace_bytes", "es_solve_device", "es_solve",
           "es_solution_rows", "es_solution_cols", "es_solution_get", "es_solution_info",
           "es_solution_free", "es_solution_modulus_bits", "es_set_gpu_reconstruction", "es_set_blocked_inverse",
           "es_set_lift_record_steps",
           "es_last_timings", "es_set_profiling", "es_kernel_profile",
           "es_batched_inverse", "es_batched_inverse_noalloc", "es_noalloc_max_n", "es_lift_digits",
           "es_reconstruct"]

_lib = None

c_i64p = ctypes.POINTER(ctypes.c_int64)
c_u64p = ctypes.POINTER(ctypes.c_uint64)
c_i32p = ctypes.POINTER(ctypes.c_int32)
c_vp = ctypes.c_void_p


class LibraryMissing(RuntimeError):
    pass


def load():
    """Load the HIP library (raises LibraryMissing if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} not found: run __graft_entry__.build() "
                             "(or python dixon_adic_lifting_amd/build.py) first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.es_strerror.argtypes = [ctypes.c_int]
    lib.es_strerror.restype = ctypes.c_char_p
    lib.es_primes.argtypes = [c_i32p, ctypes.c_int32]
    lib.es_primes.restype = ctypes.c_int
    lib.es_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.es_workspace_bytes.restype = ctypes.c_size_t
    lib.es_solve_device.argtypes = [c_vp, c_vp, ctypes.c_int32, ctypes.c_int32, c_vp, ctypes.c_size_t,
                                    c_vp, ctypes.POINTER(c_vp)]
    lib.es_solve_device.restype = ctypes.c_int
    lib.es_solve.argtypes = [c_i64p, c_i64p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(c_vp)]
    lib.es_solve.restype = ctypes.c_int
    lib.es_solution_rows.argtypes = [c_vp]
    lib.es_solution_rows.restype = ctypes.c_int32
    lib.es_solution_cols.argtypes = [c_vp]
    lib.es_solution_cols.restype = ctypes.c_int32
    lib.es_solution_get.argtypes = [c_vp, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(c_u64p), c_i32p, ctypes.POINTER(c_u64p), c_i32p]
    lib.es_solution_get.restype = ctypes.c_int
    lib.es_solution_info.argtypes = [c_vp, c_i32p, c_i32p, c_i32p, c_i32p]
    lib.es_solution_info.restype = ctypes.c_int
    lib.es_solution_free.argtypes = [c_vp]
    lib.es_solution_free.restype = None
    lib.es_solution_modulus_bits.argtypes = [c_vp]
    lib.es_solution_modulus_bits.restype = ctypes.c_int32
    lib.es_last_timings.argtypes = [ctypes.POINTER(ctypes.c_double)]
    lib.es_last_timings.restype = ctypes.c_int
    lib.es_set_blocked_inverse.argtypes = [ctypes.c_int]
    lib.es_set_blocked_inverse.restype = ctypes.c_int
    lib.es_set_lift_record_steps.argtypes = [ctypes.c_int32]
    lib.es_set_lift_record_steps.restype = ctypes.c_int
    lib.es_set_gpu_reconstruction.argtypes = [ctypes.c_int]
    lib.es_set_gpu_reconstruction.restype = ctypes.c_int
    lib.es_set_profiling.argtypes = [ctypes.c_int]
    lib.es_set_profiling.restype = ctypes.c_int
    lib.es_kernel_profile.argtypes = [ctypes.POINTER(ctypes.c_double), c_i32p, ctypes.c_int32]
    lib.es_kernel_profile.restype = ctypes.c_int
    lib.es_batched_inverse.argtypes = [c_vp, ctypes.c_int32, c_vp, ctypes.c_size_t, c_vp, c_vp, c_i32p]
    lib.es_batched_inverse.restype = ctypes.c_int
    lib.es_batched_inverse_noalloc.argtypes = [c_vp, ctypes.c_int32, c_vp, c_vp, c_i32p]
    lib.es_batched_inverse_noalloc.restype = ctypes.c_int
    lib.es_noalloc_max_n.argtypes = []
    lib.es_noalloc_max_n.restype = ctypes.c_int32
    lib.es_lift_digits.argtypes = [c_vp, c_vp, ctypes.c_int32, ctypes.c_int32, c_vp, ctypes.c_size_t, c_vp,
                                   ctypes.c_int32, c_i64p, ctypes.c_size_t, c_u64p, c_i32p]
    lib.es_lift_digits.restype = ctypes.c_int
    lib.es_reconstruct.argtypes = [c_i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(c_vp)]
    lib.es_reconstruct.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().es_strerror(int(status)).decode()


def _limbs_to_int(ptr, length: int) -> int:
    if length == 0:
        return 0
    raw = ctypes.string_at(ptr, 8 * length)
    return int.from_bytes(raw, "little")


def read_solution(sol):
    """[n][c] (num, den) pairs from a solution handle (does not free it)."""
    lib = load()
    n, c = lib.es_solution_rows(sol), lib.es_solution_cols(sol)
    sign = ctypes.c_int()
    nump, denp = c_u64p(), c_u64p()
    nl, dl = ctypes.c_int32(), ctypes.c_int32()
    out = []
    for i in range(n):
        row = []
        for k in range(c):
            st = lib.es_solution_get(sol, i, k, ctypes.byref(sign), ctypes.byref(nump), ctypes.byref(nl),
                                     ctypes.byref(denp), ctypes.byref(dl))
            if st != ES_OK:
                raise RuntimeError(strerror(st))
            num = _limbs_to_int(nump, nl.value)
            den = _limbs_to_int(denp, dl.value)
            row.append((-num if sign.value < 0 else num, den))
        out.append(row)
    return out


def solution_info(sol):
    lib = load()
    live, m, nb, db = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    lib.es_solution_info(sol, ctypes.byref(live), ctypes.byref(m), ctypes.byref(nb), ctypes.byref(db))
    return {"live_primes": live.value, "m": m.value, "num_bound_bits": nb.value, "den_bound_bits": db.value,
            "modulus_bits": lib.es_solution_modulus_bits(sol)}


def last_recon_counts():
    """(components reconstructed alone on the host, gcds finished on the host)
    for the last GPU reconstruction on this thread; (-1, -1) if none ran."""
    a, g = ctypes.c_int64(), ctypes.c_int64()
    load().es_dbg_last_recon_counts(ctypes.byref(a), ctypes.byref(g))
    return a.value, g.value


def last_timings():
    buf = (ctypes.c_double * 5)()
    load().es_last_timings(buf)
    return {"checks_ms": buf[0], "inverse_ms": buf[1], "lift_ms": buf[2], "recon_gpu_ms": buf[3],
            "reconstruct_ms": buf[4]}


KERNEL_CLASSES = ["gj_step", "lift_contract", "crt", "residual", "residues", "recon_gemm", "recon_other",
                  "recon_gcd", "gj_panel", "gj_update"]


def set_blocked_inverse(on: bool):
    """Blocked elimination with MFMA updates (default) or one launch per step, for this thread."""
    load().es_set_blocked_inverse(1 if on else 0)


def set_lift_record_steps(steps: int):
    """Lift steps whose CRT records are held before one launch forms their digits (0: default), for this thread."""
    st = load().es_set_lift_record_steps(int(steps))
    if st != 0:
        raise ValueError(strerror(st))


def set_gpu_reconstruction(on: bool):
    """Reconstruct on the GPU (default) or on the host, for this thread."""
    load().es_set_gpu_reconstruction(1 if on else 0)


def set_profiling(on: bool):
    load().es_set_profiling(1 if on else 0)


def kernel_profile():
    """{class: (total_ms, launches)} for the last solve on this thread (profiling on)."""
    ms = (ctypes.c_double * 16)()
    cnt = (ctypes.c_int32 * 16)()
    k = load().es_kernel_profile(ms, cnt, 16)
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(min(k, len(KERNEL_CLASSES)))}
