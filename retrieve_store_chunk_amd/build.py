"""Builds retrieve_store_chunk_amd/libhkv.so (gfx950) with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhkv.so")

SOURCES = ["hkv_plan.cpp", "hkv_groups.cpp", "hkv_keys.cpp", "hkv_api.cpp", "hkv_copy.hip"]
# The INT8 codec takes integer decisions in fp32 on both the GPU and the CPU
# oracle: keep IEEE division and fp32 denormals explicit.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra_flags, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
