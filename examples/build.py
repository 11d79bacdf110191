"""Builds examples/roundtrip (a store/retrieve round trip through the C ABI,
host code only) with hipcc, linked against retrieve_store_chunk_amd/libhkv.so
(found at run time relative to the binary)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "roundtrip")
    tmp = out + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "roundtrip.cpp"),
           "-L", os.path.join(ROOT, "retrieve_store_chunk_amd"), "-lhkv",
           "-Wl,-rpath,$ORIGIN/../retrieve_store_chunk_amd", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
