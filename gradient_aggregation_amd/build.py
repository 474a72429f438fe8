"""Build libgradagg.so (HIP, gfx950) in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgradagg.so")
SOURCES = ["abi.hip", "buckets.hip", "dense.hip", "variants.hip", "norm.hip", "topk.hip", "gather.hip", "history.hip", "noalloc.hip", "pack.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # one rounding per binary32 operation, as the method specifies
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _jobs() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, s[:-4] + ".o.tmp" + tag) for s in SOURCES]

    def compile_one(i):
        cmd = [hipcc()] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)

    try:
        with ThreadPoolExecutor(max_workers=_jobs()) as ex:
            list(ex.map(compile_one, range(len(SOURCES))))
        tmp = LIB + ".tmp" + tag
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
