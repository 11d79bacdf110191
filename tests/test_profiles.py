"""The committed rocprofv3 summaries (no GPU): every command in them runs a
committed program that the profiler starts directly, with flags the
benchmark accepts, and every stored traffic figure matches the algorithmic
bytes of the launches it was taken on (within 0.1%)."""
import glob
import json
import os
import re
import shlex

import pytest

import bench
import retrieve_store_chunk_amd as hkv
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
with open(os.path.join(ROOT, ".gitignore")) as _f:
    IGNORED = {ln.strip() for ln in _f if ln.strip() and not ln.startswith("#")}


def commands(path):
    with open(path) as f:
        return [ln.strip() for ln in f if ln.strip().startswith("rocprofv3 ")]


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_profile_commands_run_the_benchmark_with_valid_flags(path):
    cmds = commands(path)
    assert cmds, f"{os.path.basename(path)} names no rocprofv3 command"
    for cmd in cmds:
        argv = shlex.split(cmd)
        assert "--" in argv, cmd
        prog = argv[argv.index("--") + 1:]
        # the program itself follows "--" (no env, shell or launcher hop)
        assert prog[:2] == ["python3", "bench.py"], cmd
        args = bench.build_parser().parse_args(prog[2:])
        W.make_config(args.config)
        # output goes to an untracked folder (one .gitignore lists), never
        # into the tracked tree
        d = argv[argv.index("-d") + 1]
        assert d.split("/")[0] + "/" in IGNORED, cmd
        pmc = [a for a in argv if a == "--pmc"]
        assert len(pmc) <= 1, cmd
        if pmc:
            counters = argv[argv.index("--pmc") + 1:argv.index("--kernel-trace")]
            assert not re.search(r"sys-trace|runtime-trace", cmd), cmd
            assert 1 <= len(counters) <= 4, cmd


TRAFFIC = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


@pytest.mark.parametrize("path", TRAFFIC, ids=os.path.basename)
def test_traffic_figures_match_the_algorithmic_bytes(path):
    with open(path) as f:
        t = json.load(f)
    name = os.path.basename(path)[len("traffic_"):-len(".json")]
    assert t["workload"] == name
    cfg = W.make_config(name)
    lay = hkv.Layout(dict(cfg.desc, tile_bytes=t.get("tile_bytes", 0),
                          max_workgroups=t.get("max_workgroups", 0)))
    info = lay.info
    kda = {L["kv_group"] for L in lay.layers if not L["is_mla"]}
    waves = W.plan_waves(cfg, info["num_blocks"], lay.G, lay.k, kda, info["block_size"],
                         info["chunk_tokens"])
    reads, writes = [], []
    for w in waves:
        if w.op == "store":
            data, objb, _ = bench.wave_bytes(lay, w)
            reads.append(data)
            writes.append(objb)
    alg_read, alg_write = sum(reads) / len(reads), sum(writes) / len(writes)
    got = t["store_gather_bytes_per_launch"]
    # the gather's name carries the INT8 head_dim suffix under the codec
    kern = next(k[:-len("_bytes_per_launch")] for k in t
                if k.startswith("hkv_store_gather") and k.endswith("_bytes_per_launch"))
    assert kern == ("hkv_store_gather_int8_d%d" % cfg.desc["kda_head_dim"]
                    if cfg.desc.get("kda_codec") else "hkv_store_gather")
    assert got == t[kern + "_bytes_per_launch"]
    assert got == pytest.approx(t[kern + "_read_bytes"] + t[kern + "_write_bytes"], abs=2)
    assert abs(t[kern + "_read_bytes"] / alg_read - 1) < 1e-3
    # every launch, the INT8 gather's included, writes its algorithmic bytes
    assert abs(t[kern + "_write_bytes"] / alg_write - 1) < 1e-3
    assert abs(got / (alg_read + alg_write) - 1) < 1e-3
    assert len(t["kernel_sha"]) == 16
