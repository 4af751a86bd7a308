"""Compile the HIP sources into ``libspec_hip.so`` (gfx950), in-tree."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspec_hip.so")
SOURCES = ["abi.hip", "ngram.hip", "alloc.hip", "verify.hip", "budget.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


PROBE_LIB = os.path.join(PKG, "libspec_probe.so")   # the benchmark's streaming-read probe, not the step


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    for srcs, out in ((SOURCES, LIB), (["probe.hip"], PROBE_LIB)):
        cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               *[os.path.join(CSRC, s) for s in srcs], "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
