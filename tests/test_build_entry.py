"""The build step must work on a fresh checkout, where no library is built
yet: it may not import the product package (which raises without libhkv.so)
before that library exists."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
sys.path.insert(0, {root!r})
import __graft_entry__ as g
mods = [g._build_module(p) for p in ("retrieve_store_chunk_amd", "workloads", "oracle", "examples")]
assert all(callable(m.build) for m in mods)
loaded = sorted(m for m in sys.modules if m.split(".")[0] in ("retrieve_store_chunk_amd", "oracle", "workloads", "examples"))
print("loaded:", loaded)
assert not loaded, loaded
"""


def test_build_modules_load_without_the_packages():
    r = subprocess.run([sys.executable, "-c", PROBE.format(root=ROOT)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
