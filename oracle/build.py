"""Builds the CPU oracle library (oracle/libhkvref.so) with gcc.

TEST INFRASTRUCTURE: the oracle is only loaded by the tests, the smoke check
and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libhkvref.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "hkvref.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
