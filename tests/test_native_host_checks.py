"""Host checks of the library's index arithmetic and call tables (no GPU).

Each program under tests/native/ is built with g++ against the library's
host sources (planner, call tables, shared kernel tables) and run; it exits
non-zero on the first violation.  See each program's header for what it
checks.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "retrieve_store_chunk_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")

PROGRAMS = {
    "xcd_order.cpp": [],
    "lane_bounds.cpp": ["hkv_plan.cpp"],
    "scratch_directory.cpp": [],
    "call_tables.cpp": ["hkv_plan.cpp", "hkv_groups.cpp"],
}


@pytest.mark.parametrize("program", sorted(PROGRAMS))
def test_native_host_check(program, tmp_path):
    exe = tmp_path / program.replace(".cpp", "")
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(NATIVE, program), *[os.path.join(CSRC, s) for s in PROGRAMS[program]],
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
