"""Builds libbdssm.so (the HIP kernels and the C ABI of include/bdssm.h) for gfx950 with
hipcc, in-tree, next to this file: every source compiled to an object in parallel, then one
link."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbdssm.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "scan_valu.hip", "block_step_mfma.hip", "block_step_lat.hip", "block_step_bw.hip",
           "prefix_mfma.hip", "graph.hip", "conv.hip"]
ARCH = "gfx950"

COMPILE = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
    # packed float32 vector instructions stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
LINK = [
    f"--offload-arch={ARCH}", "-shared", "-fPIC",
    "-Wl,--no-undefined",  # a missing symbol (e.g. a kernel's launch stub) fails the build
]


def _jobs():
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n, len(SOURCES)))


def build(verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = ["hipcc", *COMPILE, "-c", "-o", obj, os.path.join(HERE, "csrc", src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *LINK, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
