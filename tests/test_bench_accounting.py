"""The benchmark's byte accounting (no GPU): the payload and HBM bytes of a
call, counted page by page from the oracle's placement, with null pages,
partial chunks and INT8 KDA pages."""
import copy

import numpy as np
import pytest

import bench
import oracle
import retrieve_store_chunk_amd as hkv
import workloads as W


def brute(ref, w):
    N, k = ref.summary["block_size"], ref.k
    data = live = 0
    for ci in range(len(w.chunks)):
        t = N * k if w.chunk_tokens is None else int(w.chunk_tokens[ci])
        for L in ref.layers:
            for j in range(k):
                if int(w.ids[ci, L["kv_group"], j]) == W.NULL_BLOCK:
                    continue
                if L["is_mla"]:
                    rows = min(N, max(0, t - j * N))
                    data += rows * (L["page_bytes"] // N)
                    live += rows * (L["page_bytes"] // N)
                else:
                    data += L["page_bytes"]
                    live += L["obj_page_bytes"]
    return data, len(w.chunks) * (ref.summary["obj_bytes0"] + ref.summary["obj_bytes1"]), live


@pytest.mark.parametrize("name,codec", [("tiny", 0), ("tiny", 1), ("k3_tp8_holes", 0),
                                        ("k3_tp8_holes", 1), ("kl_tp1_tails", 1),
                                        ("kl_tp1_int8", 1)])
def test_wave_bytes_match_page_by_page_count(name, codec):
    cfg = copy.deepcopy(W.make_small_config(name))
    cfg.desc = dict(cfg.desc, kda_codec=codec)
    ref, lay = oracle.Layout(cfg.desc), hkv.Layout(cfg.desc)
    s = ref.summary
    kda = tuple(g for g in range(ref.G)
                if not any(L["is_mla"] for L in ref.layers if L["kv_group"] == g))
    waves = W.plan_waves(cfg, s["num_blocks"], ref.G, ref.k, kda_groups=kda,
                         block_tokens=s["block_size"], chunk_tokens=s["chunk_tokens"])
    for w in waves:
        got = bench.wave_bytes(lay, w)
        assert got == brute(ref, w)
        if not codec:
            assert got[0] == got[2]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8", "--steps", "1"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """The path has no cross-GPU step: bench.py runs on one GPU and says so
    (exit 2, before it touches torch or a device)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120, cwd=root,
                       env=dict(os.environ, **env))
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_metric_line_names_each_workload():
    """The metric line names the workload's shapes and block size; for the
    Kimi-Linear TP=1 workload it is the headline metric, word for word."""
    headline = "store+retrieve GB/s of KV/state pages (Kimi-Linear shapes, N=1888); % HBM peak"
    cfg = W.make_config("kl_tp1")
    assert bench.metric_for(cfg, 1888, on_host=False) == headline
    seen = set()
    for name in W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES:
        cfg = W.make_config(name)
        lay = oracle.Layout(cfg.desc)
        on_host = cfg.extra.get("objects") == "host"
        m = bench.metric_for(cfg, lay.summary["block_size"], on_host)
        assert f"N={lay.summary['block_size']}" in m
        assert ("host-link" in m) == on_host
        seen.add(m)
    assert len(seen) == len(W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES)


def test_ceiling_flags_parse():
    ap = bench.build_parser()
    a = ap.parse_args([])
    assert not a.no_ceilings
    a = ap.parse_args(["--no-ceilings", "--copy-ceiling"])
    assert a.no_ceilings and a.copy_ceiling


def test_noalloc_entry_refuses_the_dma_engine():
    """The no-allocation entry point runs the kernels only: a workload that
    retrieves by DMA is refused before anything is allocated."""
    from workloads.runner import GpuWorkload
    with pytest.raises(ValueError, match="kernels only"):
        GpuWorkload(W.make_config("kl_tp1_host_duplex"), entry="noalloc")
    with pytest.raises(ValueError, match="kernels only"):
        GpuWorkload(W.make_config("kl_tp1"), entry="noalloc", retrieve_engine="dma")


def test_cpu_baseline_fields_on_a_tiny_sample():
    """The oracle leg reports GB/s and chunks/s on the seeded sample, the
    threads it used and the CPUs available."""
    out = bench.cpu_baseline(W.make_config("tiny"), threads=2, min_seconds=0.05, max_seconds=0.5)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["chunks_per_s"] > 0
    assert out["cores"] == 2 and out["cores_available"] >= 1
    assert "seeded generator" in out["sample"]
