"""Builds libbdssm.so (the HIP kernels and the C ABI of include/bdssm.h) for gfx950 with
hipcc, in-tree, next to this file."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbdssm.so")
SOURCES = ["api.hip", "scan_valu.hip", "block_step_mfma.hip", "block_step_lat.hip", "block_step_bw.hip", "prefix_mfma.hip", "graph.hip", "conv.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Wl,--no-undefined",  # a missing symbol (e.g. a kernel's launch stub) fails the build
    # packed float32 vector instructions stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
