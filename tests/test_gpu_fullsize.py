"""GPU parity at the workloads' full sizes, every byte, in the launch
configuration the benchmark times (default tiles, one workgroup per tile).

The pools (16-100 GiB) are too large to copy to the host, so every expected
pool and object byte is rebuilt on the device from the seeded generator at
the oracle's placements and compared with torch.equal after every wave; INT8
codec pages are compared on the host against the oracle's codec
(tests/fullsize_check.py describes the model).
"""
import pytest

import workloads as W
from tests.fullsize_check import Checker, DeviceBuild

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _log(msg):
    print(msg, flush=True)


# Every full-size workload, the duplex one included: its waves run at once
# and are checked after both have finished, in order.
FULL_SIZE = list(W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES)


def run_every_byte(name, entry="workspace"):
    """One full-size workload through the given entry point ("workspace":
    hkv_store_chunks / hkv_retrieve_chunks; "noalloc": hkv_move_chunks_noalloc),
    every pool byte checked after every wave and every object byte."""
    from workloads.runner import GpuWorkload
    cfg = W.make_config(name)
    tag = f"[fullsize] {name}" + ("" if entry == "workspace" else f" ({entry})")
    _log(tag)
    g = GpuWorkload(cfg, objects=cfg.extra.get("objects", "device"), entry=entry)
    chk = Checker(cfg, g, DeviceBuild())
    g.init_pool()
    obj_seed = W.derive_seed(cfg.seed, 77)
    g.fill_objects(obj_seed)
    chk.set_object_fill(obj_seed)
    chk.prefilled = {rc for w in g.waves if w.op == "retrieve" and w.prefilled_objects
                     for rc in w.chunks}
    g.synchronize()

    def on_wave(i, w):
        chk.on_wave(i, w)
        _log(f"{tag}: wave {i} ({w.op}, {len(w.chunks)} chunks) matches")

    g.run_all(on_wave=on_wave)
    g.synchronize()
    chk.check_objects(sorted(g.slot_of.values()), "end of run")
    s = chk.stats
    pool_total = g.pool.numel()
    obj_total = sum(g.objs[o].numel() for o in range(chk.ref.O))
    assert s["pool_bytes"] == s["waves"] * pool_total
    _log(f"{tag}: {s['waves']} waves; every pool byte compared after every wave "
         f"({pool_total / 1e9:.1f} GB each), {s['obj_bytes'] / 1e9:.1f} GB of object bytes "
         f"compared (all {obj_total / 1e9:.1f} GB at the end), {s['codec_pages']} INT8 pages "
         f"against the oracle's codec")
    chk.pool_exec.shutdown()
    del g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_every_byte(name):
    run_every_byte(name)
