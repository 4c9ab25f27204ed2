"""Build the HIP library ``libexact_solve.so`` in place (gfx950).

Every kernel is compiled for gfx950 only.  Packed fp32 instructions are
switched off for device code (``-Xclang -target-feature -Xclang
-packed-fp32-ops``); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libexact_solve.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["kernels.hip", "recon.hip"]
# per-source device flags: the gcd kernel's limb arrays (up to 64 registers,
# indexed by wave-uniform slot numbers) stay in registers only with a higher
# promotion limit than the default, which sends them to scratch at 1024
# threads per block
SOURCE_FLAGS = {"recon.hip": ["-mllvm", "-amdgpu-promote-alloca-to-vector-limit=1024"]}
HOST_SOURCES = ["api.cpp", "host.cpp", "bignum.cpp", "debug.cpp", "recon_host.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{CSRC}",
          f"-I{os.path.join(os.path.dirname(HERE), 'include')}"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-pthread"])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
