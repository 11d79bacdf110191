"""Builds workloads/libhkvfill.so (GPU fill of seeded inputs) and
workloads/libhkvceiling.so (HBM reference-rate kernels for bench.py)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libhkvfill.so")
CEILING_LIB = os.path.join(HERE, "libhkvceiling.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = ["hipcc", *HIP_FLAGS, os.path.join(HERE, src), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """The GPU fill of seeded inputs and the HBM reference-rate kernels."""
    _hipcc("fill.hip", LIB, verbose)
    _hipcc("hbm_ceiling.hip", CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
