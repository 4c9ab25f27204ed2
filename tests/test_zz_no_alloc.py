"""The batched inverse through es_batched_inverse_noalloc, the entry point
for callers that cannot allocate (fixed device scratch, no workspace),
against es_batched_inverse, the entry point that takes a workspace.

Two calls in a row, the second with a smaller, ragged input, so the second
must not depend on what the first left in the shared scratch: the live
primes' inverses must be identical bit for bit and the singular-prime flags
identical; neither call may change torch's allocations or the device's free
memory; and n above the scratch's limit is rejected before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import dixon_adic_lifting_amd as es
from dixon_adic_lifting_amd import _lib, workloads as W

pytestmark = pytest.mark.gpu


def noalloc_call(dA, n, out):
    lib = _lib.load()
    flags = (ctypes.c_int32 * _lib.NUM_PRIMES)()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.es_batched_inverse_noalloc(ctypes.c_void_p(dA.data_ptr()), n, stream, ctypes.c_void_p(out.data_ptr()),
                                        flags)
    return st, list(flags)


def test_noalloc_inverse_matches_the_workspace_entry_point():
    assert es.noalloc_max_n() == 512
    for n, seed in [(300, 41), (97, 42)]:
        A, _ = W.uniform_system(n, 1, 24, seed)
        A[0] *= 3 * 5           # det A divisible by 3 and 5: those primes are flagged
        A[n // 2] *= 251
        dA = torch.as_tensor(A).cuda()
        Bref, fref = es.batched_inverse(dA)
        out = torch.full((_lib.NUM_PRIMES, n, n), 77, dtype=torch.int8, device="cuda")
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        alloc0 = torch.cuda.memory_allocated()
        st, flags = noalloc_call(dA, n, out)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert st == 0, _lib.strerror(st)
        assert torch.cuda.memory_allocated() == alloc0
        assert free0 - free1 < (1 << 20), (free0, free1)
        assert flags == fref
        assert flags[0] == 1 and flags[1] == 1 and flags[52] == 1 and sum(flags) < 53
        live = [j for j in range(_lib.NUM_PRIMES) if flags[j] == 0]
        assert torch.equal(out[live], Bref[live])


def test_noalloc_rejects_n_beyond_the_scratch():
    n = es.noalloc_max_n() + 1
    dA = torch.zeros((n, n), dtype=torch.int64, device="cuda")
    out = torch.zeros((1,), dtype=torch.int8, device="cuda")
    st, _ = noalloc_call(dA, n, out)
    assert st == _lib.ES_ETOOBIG
    with pytest.raises(ValueError):
        es.batched_inverse_noalloc(dA)
