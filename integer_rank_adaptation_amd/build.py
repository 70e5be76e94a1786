"""Build libintlora.so (all HIP kernels + the C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libintlora.so")
SOURCES = ["capi.hip", "merge.hip", "linear.hip", "ste.hip"]

# -ffp-contract=off: no implicit multiply-add fusion (every fp32 step is the IEEE
# operation written); packed fp32 instructions are disabled for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libintlora.so")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
