"""The C-ABI example (examples/roundtrip.cpp): a store and a retrieve through
include/hkv.h and the HIP runtime alone, run as a process of its own.  Every
stored page must come back byte for byte at its fresh block id and nothing
else in the second pool may change, through the workspace entry points and
through the no-allocation one captured into a HIP graph and replayed."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_abi_roundtrip_example():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    exe = os.path.join(ROOT, "examples", "roundtrip")
    if not os.path.exists(exe):
        from examples import build
        build.build()
    print("[c example] running examples/roundtrip", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("roundtrip ok"), r.stdout
    assert "3 replays match" in r.stdout, r.stdout
    print(r.stdout, flush=True)
