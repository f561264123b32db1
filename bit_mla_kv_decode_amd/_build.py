"""Build the gfx950 HIP library in-tree (hipcc --offload-arch=gfx950)."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_lowbit.so")
PEAKS_LIB = os.path.join(PKG, "libmla_peaks.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # bit-exact quantizer: IEEE division, no contraction, no fast-math
    "-ffp-contract=off", "-fno-fast-math",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(srcs, lib, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the decode library (csrc/*.hip -> libmla_lowbit.so) and the
    practical-peak microbenchmarks (csrc/peaks -> libmla_peaks.so); always rebuilds."""
    _hipcc(sorted(glob.glob(os.path.join(CSRC, "peaks", "*.hip"))), PEAKS_LIB, verbose)
    return _hipcc(sources(), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
