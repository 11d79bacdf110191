"""Host-side checks of the C-ABI library (no GPU needed).

- libhkv exports every function include/hkv.h declares;
- its planner gives the same layout as the oracle's for the five workloads
  and for random small layouts (including identical error codes);
- argument validation rejects bad calls before any HIP call.  These use
  fake device addresses, so they run only where no GPU is visible; the GPU
  suite repeats the error paths with real buffers.
"""
import os
import re

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import retrieve_store_chunk_amd as hkv
import workloads
from tests.test_oracle_pins import layout_params, small_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "hkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"hkv_unified_block_size", "hkv_layout_init", "hkv_store_chunks",
            "hkv_retrieve_chunks", "hkv_move_chunks_noalloc"} <= set(names)
    for n in names:
        assert hasattr(hkv.lib, n), n


PAGE_TITLES = ("Hybrid Attention Models", "Kimi-Linear", "Kimi K3",
               "vLLM hybrid KV-cache blog", "Mooncake K3 blog")


def declaration_comment(name):
    """The comment block that ends right before `name`'s declaration."""
    text = open(os.path.join(ROOT, "include", "hkv.h")).read()
    m = re.search(r"/\*((?:(?!\*/).)*)\*/\s*(?:#define[^\n]*\n\s*)*hkv_status\s+" + name +
                  r"\s*\(", text, flags=re.S)
    assert m, name
    return m.group(1)


@pytest.mark.parametrize("name", ["hkv_unified_block_size", "hkv_layout_init",
                                  "hkv_store_chunks", "hkv_retrieve_chunks"])
def test_boundary_calls_cite_the_passage_that_defines_them(name):
    comment = declaration_comment(name)
    assert any(t in comment for t in PAGE_TITLES), name


def test_every_codec_head_dim_has_its_kernel_pair():
    """The launcher runs an INT8 layout on the kernel pair built for its KDA
    head_dim, so every head_dim the planner admits under the codec needs
    both kernels in the library."""
    admitted = []
    for d in range(1, 1025):
        desc = workloads._desc([0, 1], 1, d, 8, 2, 1, 1 << 26, kda_codec=1)
        try:
            hkv.hkv_layout_destroy(hkv.hkv_layout_init(desc))
            admitted.append(d)
        except hkv.HkvError as e:
            assert e.status == hkv.HKV_E_ARG
    assert admitted == [16, 32, 64, 128, 256]
    for d in admitted:
        for kernel in ("hkv_store_gather_int8_d", "hkv_retrieve_scatter_int8_d"):
            assert hasattr(hkv.lib, f"{kernel}{d}"), f"{kernel}{d}"
    assert hasattr(hkv.lib, "hkv_store_gather") and hasattr(hkv.lib, "hkv_retrieve_scatter")


def same_plan(desc):
    ref = oracle.Layout(desc)
    got = hkv.Layout(desc)
    s, i = ref.summary, got.info
    assert i["block_size"] == s["block_size"]
    assert i["chunk_tokens"] == s["chunk_tokens"]
    assert i["blocks_per_chunk"] == s["blocks_per_chunk"]
    assert i["num_blocks"] == s["num_blocks"]
    assert i["n_layers"] == s["n_layers"]
    assert i["n_kv_groups"] == s["n_kv_groups"]
    assert i["n_obj_groups"] == s["n_obj_groups"]
    assert i["path"] == s["path"]
    assert i["n_slabs"] == s["n_slabs"]
    assert i["unified_page_bytes"] == s["unified_page_bytes"]
    assert i["block_stride"] == s["block_stride"]
    assert i["pool_bytes_used"] == s["pool_bytes_used"]
    assert i["obj_bytes"] == [s["obj_bytes0"], s["obj_bytes1"]]
    assert i["chunk_payload_bytes"] == s["obj_bytes0"] + s["obj_bytes1"]
    for a, b in zip(got.layers, ref.layers):
        for key in oracle.LAYER_FIELDS:
            assert a[key] == b[key], key
    return got


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES + workloads.EXTRA_CONFIG_NAMES)
def test_planner_matches_oracle_on_workloads(name):
    same_plan(workloads.make_config(name).desc)
    same_plan(workloads.make_small_config(name).desc)


def test_unified_block_size_matches_oracle():
    for name in workloads.CONFIG_NAMES:
        d = workloads.make_config(name).desc
        kda = oracle.kda_page_bytes(d["kda_heads"], d["kda_head_dim"], d["kda_state_bytes"],
                                    d["conv_dim"], d["conv_kernel"], d["conv_bytes"])
        n_ref = oracle.unified_block_size(kda, d["mla_width"] * d["mla_bytes"])
        assert hkv.hkv_unified_block_size(d) == n_ref
    d = workloads.make_config("kl_tp2").desc
    assert hkv.hkv_unified_block_size(d) == 944
    assert hkv.status_of(hkv.hkv_unified_block_size, d, 8) == hkv.HKV_E_ARG


def status_oracle(desc):
    try:
        oracle.Layout(desc)
        return 0
    except oracle.OracleError as e:
        return e.status


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layout_params, st.sampled_from([0, 16, 48, 64, 100]), st.integers(0, 1),
       st.sampled_from([0, 15, 16, 17, 31, 32, 100]))
def test_planner_matches_oracle_on_random_layouts(params, block_size, strict, budget):
    is_mla, path, sep, grouping, cmin, pf, conv = params
    d = small_desc(is_mla, path, sep, grouping, cmin, pf, conv_dim=conv)
    d.update(block_size=block_size, strict_chunk_multiple=strict, max_num_batched_tokens=budget)
    st_ref = status_oracle(d)
    st_got = hkv.status_of(hkv.hkv_layout_init, d)
    assert st_got == st_ref
    if st_ref == 0:
        same_plan(d)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.integers(0, 1), min_size=1, max_size=6), st.integers(1, 3),
       st.sampled_from([8, 16, 32, 48, 64, 256]), st.sampled_from([0, 4, 5, 8, 104]),
       st.sampled_from([2, 4]), st.sampled_from([0, 1, 2]), st.integers(0, 1), st.integers(0, 1),
       st.sampled_from([0, 4096, 8192, 1 << 20]))
def test_codec_layouts_match_oracle(is_mla, heads, head_dim, conv, state_bytes, codec, path, sep,
                                    tile):
    """The INT8 codec's shape rules and object layout: same status and the
    same placement (object page bytes included) as the oracle."""
    d = workloads._desc(is_mla, heads, head_dim, conv, 2, path, 1 << 30, separate=sep,
                        state_bytes=state_bytes, mla_width=64, kda_codec=codec)
    st_ref = status_oracle(d)
    assert hkv.status_of(hkv.hkv_layout_init, dict(d, tile_bytes=tile)) == st_ref
    if st_ref == 0:
        same_plan(dict(d, tile_bytes=tile))
        assert hkv.Layout(d).fingerprint() == oracle.Layout(d).fingerprint()


def test_layout_errors_match_oracle():
    base = workloads.make_config("kl_tp2").desc
    cases = [dict(block_size=928), dict(block_size=950), dict(chunk_min_tokens=0),
             dict(chunk_min_tokens=1000, strict_chunk_multiple=1), dict(pool_bytes=1000),
             dict(max_num_batched_tokens=100), dict(path=2),
             dict(kv_group_of_layer=[0] * 26 + [2]), dict(kv_group_of_layer=[-1] * 27)]
    for c in cases:
        d = dict(base, **c)
        assert hkv.status_of(hkv.hkv_layout_init, d) == status_oracle(d) != 0, c
    # knobs the oracle does not have
    for c in (dict(tile_bytes=1000), dict(tile_bytes=(1 << 30) + 4096)):
        assert hkv.status_of(hkv.hkv_layout_init, dict(base, **c)) == hkv.HKV_E_ARG


def test_workspace_size_grows_with_chunks():
    lay = hkv.Layout(workloads.make_config("kl_tp1").desc)
    a, b = lay.workspace_size(1), lay.workspace_size(1024)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    assert hkv.status_of(hkv.hkv_workspace_size, lay.handle, -1) == hkv.HKV_E_ARG


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only check")
def test_call_validation_on_host():
    lay = hkv.Layout(workloads.make_config("tiny").desc)
    G, k, O = lay.G, lay.k, lay.O
    nb = lay.info["num_blocks"]
    pool = 1 << 40
    used = lay.info["pool_bytes_used"]
    obj0 = pool + (1 << 30)
    objs = [obj0 + i * (1 << 20) for i in range(2 * O)]
    ws_bytes = lay.workspace_size(2)
    ws = pool + (1 << 32)
    ids = np.arange(2 * G * k, dtype=np.int32).reshape(2, G, k)

    def st(fn, **kw):
        a = dict(pool=pool, ids=ids, objs=objs, ws=ws, ws_bytes=ws_bytes)
        a.update(kw)
        return hkv.status_of(fn, lay.handle, a["pool"], a["ids"], a["objs"], a["ws"],
                             a["ws_bytes"], 0)

    for fn in (hkv.hkv_store_chunks, hkv.hkv_retrieve_chunks):
        assert st(fn, ws_bytes=ws_bytes - 1) == hkv.HKV_E_WORKSPACE
        assert st(fn, ws=0) == hkv.HKV_E_WORKSPACE
        assert st(fn, pool=pool + 8) == hkv.HKV_E_ALIGN
        assert st(fn, ws=ws + 4) == hkv.HKV_E_ALIGN
        assert st(fn, objs=[objs[0] + 1] + objs[1:]) == hkv.HKV_E_ALIGN
        assert st(fn, objs=[0] + objs[1:]) == hkv.HKV_E_ARG
        bad = ids.copy()
        bad[1, 0, 0] = nb
        assert st(fn, ids=bad) == hkv.HKV_E_RANGE
        bad[1, 0, 0] = -2  # -1 is HKV_NULL_BLOCK
        assert st(fn, ids=bad) == hkv.HKV_E_RANGE
        assert hkv.status_of(fn, lay.handle, pool, ids, objs, ws, ws_bytes, 0, None,
                             [1, lay.info["chunk_tokens"] + 1]) == hkv.HKV_E_ARG
        # overlapping objects / object inside the pool / workspace in the pool
        assert st(fn, objs=[objs[0]] * len(objs)) == hkv.HKV_E_ALIAS
        assert st(fn, objs=[pool + used - 256] + objs[1:]) == hkv.HKV_E_ALIAS
        assert st(fn, ws=pool) == hkv.HKV_E_ALIAS
        # an empty batch is a no-op even with NULL pointers
        assert hkv.status_of(fn, lay.handle, 0, np.zeros((0, G, k), np.int32), [], 0, 0,
                             0) == hkv.HKV_OK
    dup = ids.copy()
    dup[1, 0, 0] = dup[0, 0, 0]
    assert st(hkv.hkv_retrieve_chunks, ids=dup) == hkv.HKV_E_ALIAS
    assert hkv.status_of(hkv.hkv_store_chunks, 0, pool, ids, objs, ws, ws_bytes, 0) \
        == hkv.HKV_E_ARG
    assert "workspace" in hkv.hkv_last_error() or hkv.hkv_last_error() != ""


@pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only check")
def test_noalloc_validation_on_host():
    """hkv_move_chunks_noalloc checks its arguments like the workspace entry
    points, before any HIP call; fake addresses are safe here."""
    lay = hkv.Layout(workloads.make_config("tiny").desc)
    G, k, O = lay.G, lay.k, lay.O
    nb = lay.info["num_blocks"]
    pool = 1 << 40
    used = lay.info["pool_bytes_used"]
    objs = [pool + (1 << 30) + i * (1 << 20) for i in range(2 * O)]
    ids = np.arange(2 * G * k, dtype=np.int32).reshape(2, G, k)
    fn = hkv.hkv_move_chunks_noalloc

    def st(op, **kw):
        a = dict(pool=pool, ids=ids, objs=objs, tokens=None)
        a.update(kw)
        return hkv.status_of(fn, lay.handle, op, a["pool"], a["ids"], a["objs"], 0, None,
                             a["tokens"])

    for op in (hkv.HKV_OP_STORE, hkv.HKV_OP_RETRIEVE):
        assert st(op, pool=pool + 8) == hkv.HKV_E_ALIGN
        assert st(op, objs=[objs[0] + 1] + objs[1:]) == hkv.HKV_E_ALIGN
        assert st(op, objs=[0] + objs[1:]) == hkv.HKV_E_ARG
        bad = ids.copy()
        bad[1, 0, 0] = nb
        assert st(op, ids=bad) == hkv.HKV_E_RANGE
        assert st(op, tokens=[1, lay.info["chunk_tokens"] + 1]) == hkv.HKV_E_ARG
        assert st(op, objs=[objs[0]] * len(objs)) == hkv.HKV_E_ALIAS
        assert st(op, objs=[pool + used - 256] + objs[1:]) == hkv.HKV_E_ALIAS
        assert hkv.status_of(fn, lay.handle, op, 0, np.zeros((0, G, k), np.int32), [],
                             0) == hkv.HKV_OK
    dup = ids.copy()
    dup[1, 0, 0] = dup[0, 0, 0]
    assert st(hkv.HKV_OP_RETRIEVE, ids=dup) == hkv.HKV_E_ALIAS
    assert st(2) == hkv.HKV_E_ARG and "op must be" in hkv.hkv_last_error()
    # the DMA engine is not served (the wrapper always asks for the kernels)
    b, keep = hkv._batch(lay.handle, ids, objs, lay.info, None, hkv.HKV_ENGINE_DMA)
    import ctypes
    assert hkv.lib.hkv_move_chunks_noalloc(lay.handle, hkv.HKV_OP_RETRIEVE, pool,
                                           ctypes.byref(b), None) == hkv.HKV_E_ARG
    del keep
    # tables larger than the static scratch: k = 40 blocks per chunk at the
    # Kimi-Linear TP=1 shapes is 572,680 work items (4.6 MB of tables)
    big = hkv.Layout(dict(workloads.make_config("kl_tp1").desc, chunk_min_tokens=40 * 1888))
    bids = np.zeros((1, big.G, big.k), np.int32)
    assert hkv.status_of(fn, big.handle, hkv.HKV_OP_STORE, pool, bids, objs[:big.O], 0,
                         big.info) == hkv.HKV_E_WORKSPACE
    assert "static scratch" in hkv.hkv_last_error()


@pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only check")
def test_alias_check_cost_does_not_grow_with_the_pool():
    """A retrieve's repeated-id check sorts the call's ids: a pool of two
    billion blocks costs a small call nothing (no per-block table)."""
    import time
    desc = workloads._desc([0, 0, 0, 1], 1, 4, 4, 1, 1, 128 * (2**31 - 1), mla_width=8)
    lay = hkv.Layout(desc)
    assert lay.info["num_blocks"] == 2**31 - 1
    G, k, O = lay.G, lay.k, lay.O
    pool = 1 << 40
    objs = [(1 << 42) + i * 4096 for i in range(2 * O)]
    ids = np.array([[[2**31 - 2]], [[5]], [[2**31 - 2]], [[7]],
                    [[11]], [[13]], [[17]], [[19]]], np.int32).reshape(2, G, k)
    t0 = time.perf_counter()
    for _ in range(200):
        assert hkv.status_of(hkv.hkv_retrieve_chunks, lay.handle, pool, ids, objs, 1 << 43,
                             lay.workspace_size(2), 0) == hkv.HKV_E_ALIAS
    assert time.perf_counter() - t0 < 2.0
    assert "appears twice" in hkv.hkv_last_error()


def test_calls_past_the_item_limit_are_rejected_before_any_hip_call():
    """One call covers at most 2^31 - 1 work items (chunks x items per
    chunk); beyond that the library asks for a split, before it looks at
    any pointer (so fake addresses are safe here)."""
    lay = hkv.Layout(workloads.make_config("kl_tp1").desc)
    per_chunk_items = 14317   # 20 KDA pages of 530 tiles + 7 MLA pages of 531
    n = (2**31 - 1) // per_chunk_items + 1
    ids = np.zeros((n, lay.G, lay.k), np.int32)
    objs = [1 << 40] * (n * lay.O)
    assert hkv.status_of(hkv.hkv_store_chunks, lay.handle, 1 << 44, ids, objs, 1 << 45,
                         1 << 40, 0) == hkv.HKV_E_ARG
    assert "split" in hkv.hkv_last_error()


def test_engine_choice_is_checked_before_any_hip_call():
    """The DMA engine serves retrieves of byte-copied layouts only; other
    engine values are rejected.  These checks precede any pointer use, so
    fake addresses are safe here."""
    plain = hkv.Layout(workloads.make_config("tiny").desc)
    codec = hkv.Layout(dict(workloads.make_config("tiny").desc, kda_codec=1))
    for lay, fn, engine in ((plain, hkv.hkv_store_chunks, hkv.HKV_ENGINE_DMA),
                            (codec, hkv.hkv_retrieve_chunks, hkv.HKV_ENGINE_DMA),
                            (plain, hkv.hkv_retrieve_chunks, 2),
                            (plain, hkv.hkv_store_chunks, -1)):
        ids = np.zeros((1, lay.G, lay.k), np.int32)
        objs = [1 << 40] * lay.O
        assert hkv.status_of(fn, lay.handle, 1 << 44, ids, objs, 1 << 45, 1 << 30, 0,
                             lay.info, None, engine) == hkv.HKV_E_ARG
        assert "engine" in hkv.hkv_last_error() or "DMA" in hkv.hkv_last_error()


def test_one_hip_runtime_in_the_process():
    """libhkv must bind to the HIP runtime torch uses: two runtimes in one
    process each see the GPU alone (the second reports no device)."""
    import re
    import torch  # noqa: F401
    import workloads
    workloads._load_fill()
    maps = open("/proc/self/maps").read()
    hip = set(re.findall(r"\S*libamdhip64\S*", maps))
    hsa = set(re.findall(r"\S*libhsa-runtime64\S*", maps))
    assert len(hip) == 1, hip
    assert len(hsa) == 1, hsa


@pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only check")
def test_error_messages_are_per_thread():
    """hkv_last_error is per calling thread: eight threads failing at the same
    time for different reasons (the calls drop the interpreter lock) each
    read back their own message every time."""
    import threading
    lay = hkv.Layout(workloads.make_config("tiny").desc)
    G, k, O = lay.G, lay.k, lay.O
    nb = lay.info["num_blocks"]
    pool = 1 << 40
    objs = [pool + (1 << 30) + i * (1 << 20) for i in range(2 * O)]
    ws_bytes = lay.workspace_size(2)
    ws = pool + (1 << 32)
    ids = np.arange(2 * G * k, dtype=np.int32).reshape(2, G, k)
    bad = ids.copy()
    bad[1, 0, 0] = nb
    cases = [(dict(ids=bad), hkv.HKV_E_RANGE, f"block id {nb} outside"),
             (dict(pool=pool + 8), hkv.HKV_E_ALIGN, "pool pointer is not 16-byte aligned"),
             (dict(ws_bytes=16), hkv.HKV_E_WORKSPACE, "workspace needs"),
             (dict(objs=[objs[0]] * len(objs)), hkv.HKV_E_ALIAS, "overlaps")]
    start = threading.Barrier(8)
    failures = []

    def worker(i):
        kw, want, text = cases[i % len(cases)]
        a = dict(pool=pool, ids=ids, objs=objs, ws=ws, ws_bytes=ws_bytes)
        a.update(kw)
        fn = hkv.hkv_store_chunks if i % 2 else hkv.hkv_retrieve_chunks
        start.wait()
        for _ in range(2000):
            try:
                fn(lay.handle, a["pool"], a["ids"], a["objs"], a["ws"], a["ws_bytes"], 0)
                failures.append((i, "no error"))
                return
            except hkv.HkvError as e:
                if e.status != want or text not in str(e):
                    failures.append((i, str(e)))
                    return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:4]


def test_trace_names_the_block_size():
    """HKV_TRACE=1: the layout's block size and chunk size on stderr, like
    the engine's own line naming the block size it settled on."""
    import subprocess
    import sys
    code = ("import workloads, retrieve_store_chunk_amd as hkv; "
            "hkv.Layout(workloads.make_config('kl_tp1').desc); "
            "hkv.Layout(workloads.make_config('k3_tp8').desc)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, cwd=ROOT, env=dict(os.environ, HKV_TRACE="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "block size N=1888 tokens, chunk C=1888 (k=1), path B" in r.stderr
    assert "block size N=768 tokens, chunk C=1536 (k=2), path A" in r.stderr
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, cwd=ROOT, env=dict(os.environ, HKV_TRACE="0"))
    assert "[hkv]" not in r.stderr
