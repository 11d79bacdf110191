"""CPU: the host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

- The oracle (oracle/hkvref.c) is built with both sanitizers, and its pins
  (block size, chunk rule, layouts, store/retrieve invariants, brute force,
  codec and chunk keys) run against that build in a child process with the
  ASan runtime preloaded.
- The host programs under tests/native/ are built with both sanitizers
  against the library's host sources and run: the index replay of the
  kernels, the call tables (inline packing, grouped retrieve, DMA runs), the
  XCD order, and the C ABI's planning, queries and argument checks
  (api_checks.cpp, which also builds hkv_api.cpp and hkv_keys.cpp).
Any sanitizer report ends the program with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "retrieve_store_chunk_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

PROGRAMS = {
    "xcd_order.cpp": [],
    "lane_bounds.cpp": ["hkv_plan.cpp"],
    "scratch_directory.cpp": [],
    "call_tables.cpp": ["hkv_plan.cpp", "hkv_groups.cpp"],
    "api_checks.cpp": ["hkv_api.cpp", "hkv_plan.cpp", "hkv_groups.cpp", "hkv_keys.cpp"],
}


def _asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


@pytest.mark.parametrize("program", sorted(PROGRAMS))
def test_native_program_under_sanitizers(program, tmp_path):
    exe = tmp_path / program.replace(".cpp", "")
    hip = []
    if program == "api_checks.cpp":
        # hkv_api.cpp calls the HIP runtime (never reached by these checks)
        hip = ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-L", "/opt/rocm/lib",
               "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    cmd = ["g++", "-std=c++17", "-Wall", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(NATIVE, program), *[os.path.join(CSRC, s) for s in PROGRAMS[program]],
           *hip, "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900, env=ENV)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "libhkvref_san.so"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared", *SAN,
                    os.path.join(ROOT, "oracle", "hkvref.c"), "-o", str(lib), "-lm"], check=True)
    probe = ("import sys, oracle; oracle.lib(); "
             "assert 'libhkvref_san' in open('/proc/self/maps').read(), 'sanitized oracle not loaded'; "
             "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
             "'tests/test_oracle_pins.py', 'tests/test_codec.py', 'tests/test_keys.py']))")
    env = dict(ENV, HKVREF_LIB=str(lib), LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0")  # the interpreter itself is not leak-clean
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True,
                       timeout=900, cwd=ROOT, env=env)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
