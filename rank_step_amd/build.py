"""Build librank_step.so in-tree with hipcc for gfx950.

    python -m rank_step_amd.build

Every source is compiled on each call (no staleness checks); the library is
written to a temporary name and renamed into place, so a failed build never
leaves a half-written library behind.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librank_step.so")

SOURCES = ["rank_step.hip", "layout.cpp", "common.cpp"]

# IEEE-correct fp32 division and square root, denormals kept, FMA only where
# the source writes it, and no packed-fp32 instructions.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librank_step.so)")


def build(verbose=False):
    cc = hipcc()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc] + FLAGS + ["-shared", "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless.
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
