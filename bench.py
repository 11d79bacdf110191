"""Store+retrieve throughput of KV/state pages on one MI355X.

One step is one pass of the whole hot path over one batch: every wave of the
workload (for the Kimi-Linear TP=1 workload: store 1024 chunks = 128 requests
x 8 chunks of 1888 tokens, then retrieve the first 4 chunks of every request
into freshly drawn, fragmented block ids).  Inputs (pool, objects, block
tables) are seeded, synthetic and resident in HBM before timing starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
HOST_LINK_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)
HOST_SHARE_THREADS = 16  # host threads per GPU of the machine (the CPU leg's cap)
CSRC = os.path.join(ROOT, "retrieve_store_chunk_amd", "csrc")
KERNEL_SOURCES = ("hkv_copy.hip", "hkv_device_tables.hpp", "hkv_launch.hpp", "hkv_plan.cpp")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def metric_for(cfg, block_size: int, on_host: bool) -> str:
    """The metric line of a workload: its shapes and block size, against HBM
    peak (or the host link's, for objects in pinned host memory).  For the
    Kimi-Linear TP=1 workload this is the headline metric."""
    peak = "% host-link peak" if on_host else "% HBM peak"
    return f"store+retrieve GB/s of KV/state pages ({cfg.shapes}, N={block_size}); {peak}"


def kernel_source_sha() -> str:
    """Hash of the sources that decide what the copy kernels do per launch:
    the kernels, their shared tables and launch header, and the planner that
    lays out the work items."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(config: str, tile: int, max_wg: int):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    and launch configuration; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if (t.get("kernel_sha") != kernel_source_sha() or t.get("tile_bytes", 0) != tile
            or t.get("max_workgroups", 0) != max_wg):
        return None
    return t.get("store_gather_bytes_per_launch")


def wave_bytes(layout, w) -> tuple:
    """(data bytes, object bytes, live object bytes) of one call.  Data bytes
    are pool page bytes that hold data: every real byte of a page, none for a
    null id, and for an MLA page of a partial chunk the rows of its valid
    tokens.  Object bytes are the chunks' whole objects (a store writes all of
    them; what has no data behind it is zero-filled).  Live object bytes are
    the object bytes behind the data bytes: the same count, except for KDA
    pages in INT8 form, which take their smaller object page size."""
    import numpy as np
    info = layout.info
    N, k, n = info["block_size"], info["blocks_per_chunk"], len(w.chunks)
    data = live = 0
    for L in layout.layers:
        present = w.ids[:, L["kv_group"], :] != -1
        if L["is_mla"] and w.chunk_tokens is not None:
            rows = np.clip(w.chunk_tokens.astype(np.int64)[:, None] - np.arange(k) * N, 0, N)
            per = rows * (L["page_bytes"] // N)
        else:
            per = np.full((n, k), L["page_bytes"], dtype=np.int64)
        data += int((per * present).sum())
        if L["obj_page_bytes"] != L["page_bytes"]:
            per = np.full((n, k), L["obj_page_bytes"], dtype=np.int64)
        live += int((per * present).sum())
    return data, n * info["chunk_payload_bytes"], live


def cpu_available() -> int:
    """The CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_threads() -> int:
    """Host threads for the threaded oracle leg: every CPU this process may
    use, at most one GPU's share of the host (HOST_SHARE_THREADS)."""
    return max(1, min(HOST_SHARE_THREADS, cpu_available()))


def seeded_fill(arrays, seeds, threads: int) -> None:
    """Fills each uint8 array with its seed's counter-based stream (the same
    generator as the GPU inputs), in 64 MiB pieces on `threads` threads."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads as W
    piece = 64 << 20
    jobs = [(a, seed, lo) for a, seed in zip(arrays, seeds) for lo in range(0, a.size, piece)]

    def run(job):
        a, seed, lo = job
        hi = min(a.size, lo + piece)
        a[lo:hi] = W.fill_bytes(seed, lo, hi - lo)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(run, jobs))


def cpu_baseline(cfg, threads: int = 1, min_seconds: float = 10.0,
                 max_seconds: float = 30.0) -> dict:
    """The oracle (plain C, one memcpy per page, or its INT8 codec loop for
    KDA pages when the layout has one) on a bounded sample of the same
    workload: the same layout shapes in a smaller pool, 64 chunks stored and
    their first halves retrieved into fresh ids, repeated until at least
    min_seconds of wall time.  With threads > 1 the unchanged oracle runs on
    that many host threads, each storing (then retrieving) its own slice of
    the chunks; ctypes releases the GIL inside the calls."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    import workloads as W

    desc = dict(cfg.desc)
    lay_full = oracle.Layout(desc)
    per_block = lay_full.summary["pool_bytes_used"] // lay_full.summary["num_blocks"]
    n_store = 64
    ids_per_chunk = lay_full.G * lay_full.k
    desc["pool_bytes"] = per_block * (n_store * ids_per_chunk + 1)
    lay = oracle.Layout(desc)
    s = lay.summary
    # seeded bytes from the inputs' generator (the pool's and the objects'
    # streams of the workload's seed)
    pool = np.empty(s["pool_bytes_used"], np.uint8)
    objs = [[np.empty(lay.obj_bytes(o), np.uint8) for o in range(lay.O)]
            for _ in range(n_store)]
    seeded_fill([pool] + [a for row in objs for a in row],
                [W.initial_pool_seed(cfg)] + [W.derive_seed(W.object_seed(cfg, 0, c), o)
                                              for c in range(n_store) for o in range(lay.O)],
                cpu_threads())
    perm = W.permutation(W.derive_seed(cfg.seed, 1234), s["num_blocks"])
    store_ids = perm[: n_store * ids_per_chunk].reshape(n_store, lay.G, lay.k)
    perm2 = W.permutation(W.derive_seed(cfg.seed, 1235), s["num_blocks"])
    n_ret = n_store // 2
    ret_ids = perm2[: n_ret * ids_per_chunk].reshape(n_ret, lay.G, lay.k)
    # pool page bytes per chunk (the objects' size, unless KDA pages are INT8)
    payload = (n_store + n_ret) * lay.k * sum(L["page_bytes"] for L in lay.layers)
    threads = max(1, min(threads, n_ret))
    st_parts = np.array_split(np.arange(n_store), threads)
    rt_parts = np.array_split(np.arange(n_ret), threads)

    def store_part(ix):
        lay.store(pool, store_ids[ix], [objs[i] for i in ix])

    def retrieve_part(ix):
        lay.retrieve(pool, ret_ids[ix], [objs[i] for i in ix])

    passes, t_wall = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while t_wall < min_seconds and (passes == 0 or t_wall + t_wall / passes < max_seconds):
            c0 = time.perf_counter()
            if threads == 1:
                lay.store(pool, store_ids, objs)
                lay.retrieve(pool, ret_ids, objs[:n_ret])
            else:
                list(ex.map(store_part, st_parts))
                list(ex.map(retrieve_part, rt_parts))
            t_wall += time.perf_counter() - c0
            passes += 1
    gbs = passes * payload / t_wall / 1e9
    how = "single-threaded" if threads == 1 else f"{threads} host threads, chunks split evenly"
    return {"value": round(gbs, 3), "unit": "GB/s",
            "chunks_per_s": round(passes * (n_store + n_ret) / t_wall, 1), "cores": threads,
            "cores_available": cpu_available(), "kind": "oracle",
            "sample": f"{passes} passes of: store {n_store} chunks + retrieve {n_ret} chunks "
                      f"(same page shapes, pool of {s['num_blocks']} blocks, pool and object "
                      f"bytes from the workload's seeded generator); "
                      f"{passes * payload / 1e9:.1f} GB moved in {t_wall:.1f} s wall, "
                      f"{how}, plain C memcpy"
                      + (" + per-row INT8 codec of KDA pages" if s["kda_codec"] else "")}


def hbm_ceiling(buf, stream, reps: int = 10) -> dict:
    """Pure read, pure write and contiguous copy of 16 GiB halves of `buf`
    with kernels shaped like the library's (workloads/hbm_ceiling.hip)."""
    import ctypes

    import torch
    import workloads as W
    L = ctypes.CDLL(os.path.join(os.path.dirname(W.__file__), "libhkvceiling.so"))
    L.hkvceiling_launch.restype = ctypes.c_int
    L.hkvceiling_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    n = min(16 << 30, (buf.numel() // 2) // 4096 * 4096)
    if n < (1 << 30):
        return {"skipped": "needs a pool of at least 2 GiB"}
    src, dst = buf[:n], buf[n:2 * n]
    out = torch.empty(n // 4096 * 4, dtype=torch.uint8, device=buf.device)
    res = {"bytes": n}
    for kind, name, traffic in ((0, "read", n), (1, "write", n), (2, "copy", 2 * n)):
        def launch():
            rc = L.hkvceiling_launch(kind, src.data_ptr(), dst.data_ptr(), out.data_ptr(), n,
                                     stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"hbm ceiling launch failed: HIP error {rc}")
        launch()
        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name + "_GBs"] = round(traffic / (ms / 1e3) / 1e9, 1)
    res["what"] = ("4 KiB tile per 128-thread workgroup, XCD order, 16-byte nontemporal "
                   "accesses; copy = one contiguous buffer into another")
    return res


def host_link_ceiling(stream, reps: int = 3) -> dict:
    """DMA copies of 4 GiB between pinned host memory and HBM (torch copy_):
    each direction alone, then both at once on two streams."""
    import torch
    n = 4 << 30
    dev = torch.empty(n, dtype=torch.uint8, device="cuda")
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dev2 = torch.empty(n, dtype=torch.uint8, device="cuda")
    host2 = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    res = {"bytes": n}
    with torch.cuda.stream(stream):
        for name, fn in (("device_to_host", lambda: host.copy_(dev, non_blocking=True)),
                         ("host_to_device", lambda: dev.copy_(host, non_blocking=True))):
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            e1.synchronize()
            res[name + "_GBs"] = round(n / (e0.elapsed_time(e1) / reps / 1e3) / 1e9, 1)
    other = torch.cuda.Stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        with torch.cuda.stream(stream):
            host.copy_(dev, non_blocking=True)
        with torch.cuda.stream(other):
            dev2.copy_(host2, non_blocking=True)
    torch.cuda.synchronize()
    res["both_directions_GBs"] = round(2 * n * reps / (time.perf_counter() - t0) / 1e9, 1)
    del dev, host, dev2, host2
    return res


def chunk_keys_timing(g, cfg, tokens_per_request: int = 16384) -> dict:
    """Host time of hkv_chunk_keys for every request of the step: seeded
    synthetic token ids, one call per request, hash blocks of N tokens."""
    import numpy as np
    import workloads as W
    n_req = len(cfg.requests)
    rng = np.random.default_rng(W.derive_seed(cfg.seed, 31337) % (1 << 32))
    toks = rng.integers(0, 163840, (n_req, tokens_per_request), dtype=np.int64).astype(np.int32)
    g.layout.chunk_keys(toks[0])  # warm
    t0 = time.perf_counter()
    n_keys = 0
    for r in range(n_req):
        _, keys = g.layout.chunk_keys(toks[r], rank_tag=(1 << 32) | 0)
        n_keys += keys.size
    dt = time.perf_counter() - t0
    return {"requests": n_req, "tokens": int(toks.size), "keys": n_keys,
            "ms": round(dt * 1e3, 3), "Mtokens_per_s": round(toks.size / dt / 1e6, 1),
            "what": "host, one thread, one call per request (hash blocks of N tokens)"}


def build_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="kl_tp1",
                    help="workload: tiny, kl_tp2, kl_tp1 (default), k3_tp8, long_ctx, "
                         "kl_tp1_host (objects in pinned host memory), k3_tp8_holes, "
                         "kl_tp1_tails, kl_tp1_int8 (INT8 KDA objects), kl_tp1_host_duplex "
                         "(host objects, a store and a retrieve at once on two streams), "
                         "kl_tp1_int8_host (INT8 KDA objects in pinned host memory)")
    ap.add_argument("--tile-bytes", type=int, default=0)
    ap.add_argument("--retrieve-engine", choices=("kernel", "dma"), default=None,
                    help="retrieves by the scatter kernel or by DMA copies of page runs "
                         "(default: the workload's choice, else the kernel)")
    ap.add_argument("--max-workgroups", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--entry", choices=("workspace", "noalloc"), default="workspace",
                    help="the calls timed: hkv_store_chunks / hkv_retrieve_chunks with a "
                         "workspace (default), or hkv_move_chunks_noalloc (kernel engine; a "
                         "call whose tables exceed one launch's kernel arguments is split "
                         "into several launches, timed together)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step's calls into a HIP graph after the warm-up and "
                         "time its replays (one-stream workloads only; with the workspace "
                         "entry points every call's tables must fit in its kernel arguments, "
                         "with --entry noalloc any call can be captured)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the reference rates timed after the steps by default: torch "
                         "copy_ of one 8 GiB buffer (the achievable device copy, also the "
                         "plain copy kernel of known size that calibrates the rocprofv3 byte "
                         "counters) and pure-read, pure-write and contiguous-copy kernels "
                         "built like the library's")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time the torch copy_ reference even with --no-ceilings")
    ap.add_argument("--host-link-ceiling", action="store_true",
                    help="also time 4 GiB DMA copies between pinned host memory and HBM "
                         "(host-link reference rates)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="time the library-shaped read/write/copy references even with "
                         "--no-ceilings")
    return ap


def main() -> int:
    args = build_parser().parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the store/retrieve path has no cross-GPU "
              "step (each rank stores and retrieves its own shard); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch
    import workloads as W
    from workloads.runner import GpuWorkload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    cfg = W.make_config(args.config)
    log(f"workload {cfg.name}: {cfg.title}")
    objects_on = cfg.extra.get("objects", "device")
    engine = args.retrieve_engine or cfg.extra.get("retrieve_engine", "kernel")
    if args.entry == "noalloc" and engine == "dma":
        print(f"--entry noalloc runs the kernel engine only; {cfg.name} would retrieve by DMA "
              f"(pass --retrieve-engine kernel)", file=sys.stderr)
        return 2
    g = GpuWorkload(cfg, tile_bytes=args.tile_bytes, max_workgroups=args.max_workgroups,
                    objects=objects_on, retrieve_engine=args.retrieve_engine, entry=args.entry)
    info = g.info
    log(f"layout: N={info['block_size']} C={info['chunk_tokens']} k={info['blocks_per_chunk']} "
        f"blocks={info['num_blocks']} stride={info['block_stride']} "
        f"chunk payload={info['chunk_payload_bytes']} B; {len(g.waves)} waves")
    g.init_pool()
    g.fill_objects(W.derive_seed(cfg.seed, 77))
    g.prefill_objects()
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    stream = g.stream
    n_w = len(g.waves)
    on_host = objects_on == "host"
    # payload = pool page bytes that hold data; HBM traffic: a store reads the
    # data and writes whole objects, a retrieve reads the live object bytes
    # and writes the data; with host objects the object side crosses the host
    # link instead of HBM
    per_wave_payload, per_wave_hbm, per_wave_link = [], [], []
    for w in g.waves:
        data, objb, live = wave_bytes(g.layout, w)
        per_wave_payload.append(data)
        obj_side = objb if w.op == "store" else live
        per_wave_hbm.append(data if on_host else data + obj_side)
        per_wave_link.append(obj_side if on_host else 0)
    step_payload = sum(per_wave_payload)
    step_hbm = sum(per_wave_hbm)

    def one_step(events=None):
        # a duplex workload's retrieves run on a second stream, beside its stores
        for i, w in enumerate(g.waves):
            if events is not None:
                events[i][0].record(g.stream_of(w))
            g.run_wave(w)
            if events is not None:
                events[i][1].record(g.stream_of(w))

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    graph = None
    if args.graph:
        # the warm-up made each call's first, uncapturable, table upload
        if g.duplex:
            print("--graph: a duplex workload runs on two streams", file=sys.stderr)
            return 2
        import retrieve_store_chunk_amd as hkv
        graph = torch.cuda.CUDAGraph()
        try:
            with torch.cuda.graph(graph, stream=stream):
                one_step()
        except hkv.HkvError as e:
            print(f"--graph: {e}", file=sys.stderr)
            return 2
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                graph.replay()
        torch.cuda.synchronize()
        log("step captured as one HIP graph")

        def timed_step(events):
            with torch.cuda.stream(stream):
                events[0][0].record(stream)
                graph.replay()
                events[0][1].record(stream)
    else:
        timed_step = one_step

    n_ev = 1 if graph is not None else n_w
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        timed_step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_payload / (ms_per_step / 1e3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} GB/s")
    # per step, from the events on the stream: first call's start to last
    # call's end (one stream; a duplex step spans two, so it has no median)
    step_ms = None
    if graph is not None:
        step_ms = [evs[s][0][0].elapsed_time(evs[s][0][1]) for s in range(args.steps)]
    elif not g.duplex:
        step_ms = [evs[s][0][0].elapsed_time(evs[s][n_w - 1][1]) for s in range(args.steps)]
    median_ms = None
    if step_ms:
        import statistics
        median_ms = statistics.median(step_ms)
        log(f"per-step median (events): {median_ms:.3f} ms")

    # per kernel (per graph replay with --graph), from the events around it
    kern = {}
    if graph is not None:
        kern["graph_replay"] = {"launches": args.steps, "hbm": step_hbm * args.steps,
                                "link": sum(per_wave_link) * args.steps,
                                "ms": sum(e[0][0].elapsed_time(e[0][1]) for e in evs)}
    # INT8 layouts run the kernel pair built for their KDA head_dim
    sfx = f"_int8_d{cfg.desc['kda_head_dim']}" if info.get("kda_codec") else ""
    for i, w in enumerate(g.waves if graph is None else ()):
        # an INT8 store into host memory runs the line-code form of the gather
        line = "_line" if (sfx and on_host) else ""
        name = ("hkv_store_gather" + sfx + line if w.op == "store" else
                "retrieve_dma_copies" if g.retrieve_engine else "hkv_retrieve_scatter" + sfx)
        ms = [evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]
        k = kern.setdefault(name, {"launches": 0, "ms": 0.0, "hbm": 0, "link": 0,
                                   "read": 0, "write": 0})
        data, objb, live = wave_bytes(g.layout, w)
        k["read"] += data if w.op == "store" else live
        k["write"] += objb if w.op == "store" else data
        k["launches"] += args.steps
        k["ms"] += sum(ms)
        k["hbm"] += per_wave_hbm[i] * args.steps
        k["link"] += per_wave_link[i] * args.steps
    kernels = {}
    for name, k in kern.items():
        avg_ms = k["ms"] / k["launches"]
        if on_host:
            link = k["link"] / k["launches"]
            kernels[name] = {"launches_per_step": k["launches"] // args.steps,
                             "avg_ms": round(avg_ms, 4),
                             "link_bytes_per_launch": int(link),
                             "link_GBs": round(link / (avg_ms / 1e3) / 1e9, 2)}
        else:
            hbm = k["hbm"] / k["launches"]
            kernels[name] = {"launches_per_step": k["launches"] // args.steps,
                             "avg_ms": round(avg_ms, 4),
                             "hbm_bytes_per_launch": int(hbm),
                             "hbm_GBs": round(hbm / (avg_ms / 1e3) / 1e9, 1)}
    unit_key = "link_bytes_per_launch" if on_host else "hbm_bytes_per_launch"
    dom = max(kernels, key=lambda n: kernels[n][unit_key] * kernels[n]["launches_per_step"])
    link_peak = HOST_LINK_PEAK_GBS * (2 if g.duplex else 1)  # the link is full duplex
    if on_host and g.duplex:
        # both directions at once: the link bytes of a step over its time
        achieved = round(sum(per_wave_link) / (ms_per_step / 1e3) / 1e9, 2)
        roofline = {"bound": "host-link", "kernel": "hkv_store_gather + hkv_retrieve_scatter "
                    "(concurrent)", "achieved": achieved, "peak": link_peak, "unit": "GB/s",
                    "frac": round(achieved / link_peak, 4), "traffic": None}
    elif on_host:
        achieved = kernels[dom]["link_GBs"]
        roofline = {"bound": "host-link", "kernel": dom, "achieved": achieved,
                    "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HOST_LINK_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = kernels[dom]["hbm_GBs"]
        # the stored counters were taken on the workspace entry points' launches
        traffic = load_traffic(args.config, args.tile_bytes, args.max_workgroups) \
            if dom.startswith("hkv_store_gather") and args.entry == "workspace" else None
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic}

    if args.entry == "noalloc":
        # a no-allocation call may be several launches; its events span them all
        roofline["timed"] = "per call"
    out = {
        "metric": metric_for(cfg, info["block_size"], on_host),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": None if median_ms is None else round(median_ms, 4),
        "value_at_median": None if median_ms is None else
        round(step_payload / (median_ms / 1e3) / 1e9, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if info.get("kda_codec") else "u8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "title": cfg.title,
                   "chunks_per_step": sum(len(w.chunks) for w in g.waves),
                   "payload_bytes_per_step": step_payload,
                   "hbm_bytes_per_step": step_hbm,
                   "block_size": info["block_size"], "chunk_tokens": info["chunk_tokens"],
                   "path": "B packed" if info["path"] else "A padded-unified",
                   "tile_bytes": args.tile_bytes, "max_workgroups": args.max_workgroups,
                   "retrieve_engine": "dma" if g.retrieve_engine else "kernel",
                   "graph": graph is not None, "entry": args.entry},
        "objects": objects_on,
        "pct_hbm_peak": None if on_host else
        round(100 * step_hbm / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
        "pct_host_link_peak": round(100 * value / link_peak, 2) if on_host else None,
        "chunks_per_s": round(sum(len(w.chunks) for w in g.waves) / (ms_per_step / 1e3), 1),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }

    if args.copy_ceiling or not args.no_ceilings:
        n = min(8 << 30, g.pool.numel() // 2)
        a, b = g.pool[:n], g.pool[n:2 * n]
        for _ in range(3):
            b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        out["copy_ceiling"] = {"bytes": n, "avg_ms": round(ms, 4),
                               "hbm_GBs": round(2 * n / (ms / 1e3) / 1e9, 1),
                               "what": "torch copy_ of one contiguous buffer (read + write)"}
        log(f"copy ceiling: {out['copy_ceiling']['hbm_GBs']} GB/s")

    out["chunk_keys"] = chunk_keys_timing(g, cfg)
    log(f"chunk keys: {out['chunk_keys']}")

    if args.host_link_ceiling:
        out["host_link_ceiling"] = host_link_ceiling(stream)
        log(f"host link reference rates: {out['host_link_ceiling']}")

    if args.hbm_ceiling or not args.no_ceilings:
        out["hbm_ceiling"] = hbm_ceiling(g.pool, stream)
        log(f"HBM reference rates: {out['hbm_ceiling']}")
        dk = kern.get(roofline["kernel"])
        if roofline["bound"] == "hbm" and dk and dk.get("read", 0) + dk.get("write", 0):
            # what this process's memory placement allows the dominant kernel:
            # its read/write mix at the library-shaped reference rates
            hc = out["hbm_ceiling"]
            rs = dk["read"] / (dk["read"] + dk["write"])
            mix = 1.0 / (rs / hc["read_GBs"] + (1.0 - rs) / hc["write_GBs"])
            roofline["process_ceiling"] = {
                "GBs": round(mix, 1), "frac": round(roofline["achieved"] / mix, 4),
                "read_share": round(rs, 4),
                "what": "the kernel's read/write mix at the read and write rates of the "
                        "library-shaped reference kernels timed in this process"}
            log(f"dominant kernel at {100 * roofline['achieved'] / mix:.1f}% of this "
                f"process's read/write mix ceiling ({mix:.0f} GB/s)")

    del g
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg)
        log(f"cpu baseline: {out['cpu_baseline']['value']} GB/s")
        nt = cpu_threads()
        if nt > 1:
            out["cpu_baseline_threads"] = cpu_baseline(cfg, threads=nt)
            out["cpu_baseline_threads"]["cores_note"] = (
                f"{cpu_available()} CPUs available to the process; at most "
                f"{HOST_SHARE_THREADS} used, one GPU's share of the host")
            log(f"cpu baseline, {nt} threads: {out['cpu_baseline_threads']['value']} GB/s")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
