"""Build libtpdecode.so in-tree: host plan code with g++, kernels with hipcc
for gfx950, linked into one shared library next to this file."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtpdecode.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

ARCH = "gfx950"
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
              "-I" + os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel, `jobs` at a time; 0 = the host's
    cores, at most 8) and link them; every call compiles everything."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    cmds, objs = [], []
    plan_o = os.path.join(BUILD, "tp_plan.o")
    cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "tp_plan.cpp"), "-o", plan_o])
    objs.append(plan_o)
    for src in sorted(os.listdir(CSRC)):
        if src.endswith(".hip"):
            o = os.path.join(BUILD, src[:-4] + ".o")
            cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", o])
            objs.append(o)
    n = jobs or max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=n) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
