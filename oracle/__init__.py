"""CPU oracle for the exact rational solver -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct CPU code that computes what the GPU path
computes, written from the exact-solve card (phanerozoic/exact-solve) and the
mathematics it rests on:

* ``exact``   -- the result's definition: x = A^-1 b over Q in lowest terms,
                 by fraction-free Bareiss elimination on Python integers
                 (the card's "Correctness" section: an exact Gaussian
                 elimination oracle; "API": None when A is singular).
* ``modular`` -- the primes below 256 and A^-1 mod q by plain Gauss-Jordan on
                 [A | I] (the card's "Method": batched modular inverse).
* ``dixon``   -- Dixon's p-adic digit recurrence with B = A^-1 mod P, the
                 Hadamard bounds that fix the step count, and Wang's rational
                 reconstruction (the card's "Method").
* ``cbareiss``-- the same Bareiss elimination in plain C with its own bignum
                 and POSIX threads, for sizes Python cannot finish.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything in this package.  It
shares no code with the HIP library in ``dixon_adic_lifting_amd``; the only
common module is the seeded input generator
(``dixon_adic_lifting_amd.workloads``), which holds none of the method.
"""
