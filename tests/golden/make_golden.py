"""Write SHA-256 digests of the oracle's exact solutions for the workloads.

Calls only ``oracle/`` (the plain-C Bareiss oracle, checked bit for bit against
the Python oracle by the CPU tests) on the seeded inputs of
``dixon_adic_lifting_amd.workloads``.  The canonical text of a solution is one
line per component in row-major order, ``"<num hex> <den hex>\\n"`` with a
leading ``-`` on negative numerators, lowest terms, positive denominators.

Usage:  python tests/golden/make_golden.py [names...] [--threads T]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from dixon_adic_lifting_amd import workloads as W  # noqa: E402
from oracle import cbareiss, exact  # noqa: E402

OUT = os.path.join(HERE, "oracle_digests.json")


def canonical_text(X) -> str:
    def h(v):
        return ("-" + format(-v, "x")) if v < 0 else format(v, "x")
    return "".join(f"{h(p)} {h(q)}\n" for row in X for (p, q) in row)


def digest(X) -> str:
    return hashlib.sha256(canonical_text(X).encode()).hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="*", default=["c1_n32_int8", "c2_pascal30", "c3_n256_int24"])
    ap.add_argument("--threads", type=int, default=cbareiss.default_threads())
    args = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in args.names:
        A, b = W.generate(name)
        t0 = time.time()
        X = cbareiss.solve(A, b, args.threads)
        secs = time.time() - t0
        assert X is not None, name
        if A.shape[0] <= 64:
            assert X == exact.solve(A, b)
        else:
            assert exact.check_solution(A, b, X)
        maxbits = max(max(abs(p).bit_length(), q.bit_length()) for row in X for (p, q) in row)
        data[name] = {"sha256": digest(X), "n": int(A.shape[0]), "c": int(b.shape[1]),
                      "max_bits": maxbits, "oracle_seconds": round(secs, 2),
                      "oracle_threads": args.threads, "oracle": "oracle/bareiss.c"}
        print(name, data[name], flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
