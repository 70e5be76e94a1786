"""Build libintlora.so (all HIP kernels + the C ABI) for gfx950, in-tree.

Each source is compiled to an object in parallel, then the objects are linked.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libintlora.so")
SOURCES = ["capi.hip", "merge.hip", "linear.hip", "ste.hip"]

# -ffp-contract=off: no implicit multiply-add fusion (every fp32 step is the IEEE
# operation written); packed fp32 instructions are disabled for all device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="intlora_build_") as tmpd:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpd, src.replace(".hip", ".o"))
            jobs.append((obj, [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
                               "-o", obj]))
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
            results = list(ex.map(lambda j: _run(j[1]), jobs))
        for (obj, cmd), (rc, msgs) in zip(jobs, results):
            if verbose:
                print(" ".join(cmd))
            if rc != 0:
                sys.stderr.write("\n".join(msgs) + "\n")
                raise RuntimeError("hipcc failed compiling " + os.path.basename(cmd[-3]))
            if verbose and msgs:
                print("\n".join(msgs))
        tmp = LIB + ".tmp%d" % os.getpid()
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in jobs]
        rc, msgs = _run(link)
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("linking libintlora.so failed")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
