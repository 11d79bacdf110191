"""GPU: hkv_move_chunks_noalloc against hkv_store_chunks / hkv_retrieve_chunks.

Every case runs the same calls through both entry points on twin buffers
(same seeded pool and object bytes) and compares the whole pool and every
object byte for byte after each call: two stores in a row, the second
smaller, then two retrieves in a row, the second smaller.  The cases cover
calls that need several launches (more chunks than one launch's kernel
arguments hold), null ids and partial chunks, the INT8 codec, and several
layouts sharing the static scratch, with evictions when they outgrow it.
The tiny workload is also checked against the oracle, full-size workloads
run through the no-allocation entry point with every byte checked, and
captured no-allocation calls replay correctly.
"""
import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _align(x, a=256):
    return (x + a - 1) // a * a


class Twin:
    """One layout, two pools and two sets of object slots with equal bytes:
    side 0 goes through the workspace entry points, side 1 through the
    no-allocation one."""

    def __init__(self, desc, n_slots, seed):
        import retrieve_store_chunk_amd as hkv
        self.hkv = hkv
        self.lay = hkv.Layout(desc)
        info = self.lay.info
        self.info = info
        self.used = info["pool_bytes_used"]
        self.obj_stride = [_align(max(1, info["obj_bytes"][o])) for o in range(self.lay.O)]
        # equal seeded bytes on both sides (the counter-based generator, on the GPU)
        self.pools = [torch.empty(_align(self.used), dtype=torch.uint8, device="cuda")
                      for _ in range(2)]
        for p in self.pools:
            W.gpu_fill(p.data_ptr(), p.numel(), W.derive_seed(seed, 1))
        self.objs = []
        for side in range(2):
            row = []
            for o in range(self.lay.O):
                a = torch.empty(n_slots * self.obj_stride[o], dtype=torch.uint8, device="cuda")
                W.gpu_fill(a.data_ptr(), a.numel(), W.derive_seed(seed, 2, o))
                row.append(a)
            self.objs.append(row)
        self.n_slots = n_slots
        self.ws_bytes = self.lay.workspace_size(n_slots)
        self.ws = torch.empty(max(256, self.ws_bytes), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()

    def ptrs(self, side, slots):
        return [self.objs[side][o].data_ptr() + s * self.obj_stride[o]
                for s in slots for o in range(self.lay.O)]

    def call(self, op, ids, slots, tokens=None, noalloc_first=True):
        """The same call on both sides, then a byte-for-byte comparison."""
        hkv = self.hkv
        s = self.stream.cuda_stream
        order = (1, 0) if noalloc_first else (0, 1)
        for side in order:
            pool = self.pools[side].data_ptr()
            if side == 1:
                code = hkv.HKV_OP_STORE if op == "store" else hkv.HKV_OP_RETRIEVE
                self.lay.move_noalloc(code, pool, ids, self.ptrs(1, slots), s,
                                      chunk_tokens=tokens)
            elif op == "store":
                self.lay.store(pool, ids, self.ptrs(0, slots), self.ws.data_ptr(),
                               self.ws_bytes, s, chunk_tokens=tokens)
            else:
                self.lay.retrieve(pool, ids, self.ptrs(0, slots), self.ws.data_ptr(),
                                  self.ws_bytes, s, chunk_tokens=tokens)
        self.stream.synchronize()
        assert torch.equal(self.pools[0], self.pools[1]), f"{op}: pools differ"
        for o in range(self.lay.O):
            assert torch.equal(self.objs[0][o], self.objs[1][o]), f"{op}: objects {o} differ"


def _ids(rng, n, G, k, num_blocks, distinct, null_frac=0.0):
    if distinct:
        ids = rng.permutation(num_blocks)[: n * G * k].astype(np.int32)
    else:
        ids = rng.integers(0, num_blocks, size=n * G * k).astype(np.int32)
    if null_frac:
        ids[rng.random(ids.size) < null_frac] = -1
    return ids.reshape(n, G, k)


def _tokens(rng, n, C, partial):
    if not partial:
        return None
    t = np.full(n, C, dtype=np.int32)
    sel = rng.random(n) < 0.5
    t[sel] = rng.integers(0, C + 1, size=int(sel.sum()))
    return t


def run_case(desc, seed, n_store, n_retrieve, null_frac=0.0, partial=False,
             store_repeats=False):
    """Store n_store[0] then n_store[1] chunks, retrieve n_retrieve[0] then
    n_retrieve[1] chunks, each call on both entry points."""
    rng = np.random.default_rng(seed)
    n_slots = max(max(n_store), max(n_retrieve))
    t = Twin(desc, n_slots, seed)
    G, k = t.lay.G, t.lay.k
    nb, C = t.info["num_blocks"], t.info["chunk_tokens"]
    _log(f"[noalloc] case seed={seed:#x} blocks={nb} G={G} k={k} store={n_store} "
         f"retrieve={n_retrieve} nulls={null_frac} partial={partial}")
    for i, n in enumerate(n_store):
        ids = _ids(rng, n, G, k, nb, distinct=not store_repeats, null_frac=null_frac)
        t.call("store", ids, list(range(n)), _tokens(rng, n, C, partial),
               noalloc_first=(i == 0))
    for i, n in enumerate(n_retrieve):
        ids = _ids(rng, n, G, k, nb, distinct=True, null_frac=null_frac)
        t.call("retrieve", ids, list(range(n)), _tokens(rng, n, C, partial),
               noalloc_first=(i == 0))
    return t


def many_blocks_desc():
    # 4 layers KKKM, 88-byte KDA pages and 128-byte MLA pages, path B: a
    # 1 MiB pool holds 8192 blocks, so one retrieve can take 2000 chunks
    # (21 launches of 96).
    return W._desc([0, 0, 0, 1], 1, 4, 4, 1, 1, 1 << 20, mla_width=8)


def codec_desc():
    # INT8 codec, head_dim 16: 2 heads x 16 x 16 fp32 + (96, 3) bf16; path B,
    # 910 blocks of 18,432 bytes.
    return W._desc([0, 0, 0, 1], 2, 16, 96, 2, 1, 16 << 20, kda_codec=1)


def test_noalloc_matches_workspace_entry_points_tiny():
    run_case(W.make_config("tiny").desc, 0x5EED01, n_store=(300, 40), n_retrieve=(16, 5),
             store_repeats=True)


def test_noalloc_kimi_linear_tp1_shapes():
    cfg = W.make_small_config("kl_tp1")
    run_case(cfg.desc, 0x5EED02, n_store=(17, 5), n_retrieve=(17, 3))


def test_noalloc_k3_holes_and_tails():
    cfg = W.make_small_config("k3_tp8_holes")
    cfg.desc["pool_bytes"] = 2 << 30  # 202 blocks: 20 chunks of 8 distinct ids
    run_case(cfg.desc, 0x5EED03, n_store=(20, 7), n_retrieve=(20, 6), null_frac=0.4,
             partial=True)


def test_noalloc_several_launches_per_call():
    run_case(many_blocks_desc(), 0x5EED04, n_store=(2000, 150), n_retrieve=(2000, 150))
    run_case(many_blocks_desc(), 0x5EED05, n_store=(700, 97), n_retrieve=(1500, 96),
             null_frac=0.2, partial=True)


def test_noalloc_int8_codec():
    run_case(codec_desc(), 0x5EED06, n_store=(200, 30), n_retrieve=(150, 20))


def test_noalloc_layouts_take_turns_on_the_scratch():
    """Alternating layouts: both stay in the scratch, each at its own range;
    results stay equal."""
    a = Twin(W.make_config("tiny").desc, 8, 0x5EED07)
    b = Twin(many_blocks_desc(), 8, 0x5EED08)
    rng = np.random.default_rng(0x5EED09)
    for step in range(3):
        for t in (a, b, a):
            nb = t.info["num_blocks"]
            t.call("store", _ids(rng, 8, t.lay.G, t.lay.k, nb, distinct=False),
                   list(range(8)))
            t.call("retrieve", _ids(rng, 3, t.lay.G, t.lay.k, nb, distinct=True), [0, 1, 2])


def test_noalloc_oracle_round_trip_tiny():
    """The no-allocation entry point alone against the oracle."""
    import retrieve_store_chunk_amd as hkv
    cfg = W.make_config("tiny")
    lay = hkv.Layout(cfg.desc)
    ref = oracle.Layout(cfg.desc)
    used = ref.summary["pool_bytes_used"]
    pool_ref = W.fill_bytes(0xABC, 0, used)
    pool = torch.from_numpy(pool_ref).to("cuda")
    rng = np.random.default_rng(0x5EED0A)
    n = 12
    ids = _ids(rng, n, ref.G, ref.k, ref.summary["num_blocks"], distinct=True)
    objs = [[torch.zeros(ref.obj_bytes(o), dtype=torch.uint8, device="cuda")
             for o in range(ref.O)] for _ in range(n)]
    objs_ref = [[np.zeros(ref.obj_bytes(o), np.uint8) for o in range(ref.O)] for _ in range(n)]
    ptrs = [objs[c][o].data_ptr() for c in range(n) for o in range(ref.O)]
    lay.move_noalloc(hkv.HKV_OP_STORE, pool.data_ptr(), ids, ptrs)
    ref.store(pool_ref, ids, objs_ref)
    ids2 = _ids(rng, n, ref.G, ref.k, ref.summary["num_blocks"], distinct=True)
    lay.move_noalloc(hkv.HKV_OP_RETRIEVE, pool.data_ptr(), ids2, ptrs)
    ref.retrieve(pool_ref, ids2, objs_ref)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), pool_ref)
    for c in range(n):
        for o in range(ref.O):
            assert np.array_equal(objs[c][o].cpu().numpy(), objs_ref[c][o])


# Full-size workloads through the no-allocation entry point alone, in the
# launch configuration the benchmark times: every pool byte after every wave
# and every object byte against the bytes rebuilt from the oracle's
# placements (the checker of the full-size parity tests).  Every workload but
# the duplex one, whose retrieves go by DMA (the entry point runs kernels).
NOALLOC_FULL_SIZE = [n for n in W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES
                     if W.make_config(n).extra.get("retrieve_engine", "kernel") == "kernel"]


@pytest.mark.parametrize("name", NOALLOC_FULL_SIZE)
def test_noalloc_full_size_every_byte(name):
    from tests.test_gpu_fullsize import run_every_byte
    run_every_byte(name, entry="noalloc")


@pytest.mark.parametrize("name", ["tiny", "kl_tp1", "k3_tp8_holes", "kl_tp1_int8_host"])
def test_noalloc_graph_capture_replays(name):
    """A no-allocation store and retrieve captured into one HIP graph, after
    one eager call has put the layout's tables in the static scratch.  Three
    replays, with new pool and object bytes written eagerly before each, all
    match the oracle applied to that replay's inputs.  With INT8 objects in
    host memory the captured store is the line-code gather."""
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    cfg = W.make_config(name) if name == "tiny" else W.make_small_config(name)
    _log(f"[noalloc graph] {name}")
    g = GpuWorkload(cfg, entry="noalloc", objects=cfg.extra.get("objects", "device"))
    ref = oracle.Layout(cfg.desc)
    calls = []
    for op in ("store", "retrieve"):
        w = next(w for w in g.waves if w.op == op)
        tok = None if w.chunk_tokens is None else w.chunk_tokens[:8].copy()
        calls.append((w.chunks[:8], w.ids[:8].copy(), tok))
    (s_chunks, s_ids, s_tok), (r_chunks, r_ids, r_tok) = calls
    P, S = g.pool.data_ptr(), g.stream
    g.init_pool()
    g.layout.move_noalloc(hkv.HKV_OP_STORE, P, s_ids, g.object_ptrs(s_chunks), S.cuda_stream,
                          chunk_tokens=s_tok)
    S.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=S):
        g.layout.move_noalloc(hkv.HKV_OP_STORE, P, s_ids, g.object_ptrs(s_chunks),
                              S.cuda_stream, chunk_tokens=s_tok)
        g.layout.move_noalloc(hkv.HKV_OP_RETRIEVE, P, r_ids, g.object_ptrs(r_chunks),
                              S.cuda_stream, chunk_tokens=r_tok)
    used = ref.summary["pool_bytes_used"]
    slots = list(dict.fromkeys(list(s_chunks) + list(r_chunks)))
    for rep in range(3):
        seed = W.derive_seed(cfg.seed, 7300 + rep)
        pool_ref = W.fill_bytes(seed, 0, used)
        g.pool[:used].copy_(torch.from_numpy(pool_ref))
        objs_ref = {}
        for i, rc in enumerate(slots):
            objs_ref[rc] = [W.fill_bytes(W.derive_seed(seed, 1 + 4 * i + o), 0, ref.obj_bytes(o))
                            for o in range(ref.O)]
            for o in range(ref.O):
                g.object_view(rc, o).copy_(torch.from_numpy(objs_ref[rc][o]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref.store(pool_ref, s_ids, [objs_ref[rc] for rc in s_chunks], chunk_tokens=s_tok)
        ref.retrieve(pool_ref, r_ids, [objs_ref[rc] for rc in r_chunks], chunk_tokens=r_tok)
        assert np.array_equal(g.host_pool()[:used], pool_ref), f"pool differs on replay {rep}"
        for rc in slots:
            for o in range(ref.O):
                assert np.array_equal(g.host_object(rc, o), objs_ref[rc][o]), \
                    f"object {rc}/{o} differs on replay {rep}"
    del graph, g
    torch.cuda.empty_cache()


def test_noalloc_capture_refuses_a_layout_not_in_the_scratch():
    """Under capture, a no-allocation call whose layout's tables are not in
    the static scratch (another layout has been used there, this one not yet)
    returns HKV_E_CAPTURE and enqueues nothing: the captured graph replays
    only the caller's own work, and the pool and objects keep their bytes."""
    import retrieve_store_chunk_amd as hkv
    a = Twin(W.make_config("tiny").desc, 4, 0x5EED0B)
    b = Twin(many_blocks_desc(), 4, 0x5EED0C)
    rng = np.random.default_rng(0x5EED0D)
    S = a.stream
    # the scratch now holds b's tables, not a's
    b.call("store", _ids(rng, 4, b.lay.G, b.lay.k, b.info["num_blocks"], distinct=True),
           list(range(4)))
    torch.cuda.synchronize()
    ids = _ids(rng, 4, a.lay.G, a.lay.k, a.info["num_blocks"], distinct=True)
    pool0 = a.pools[1].clone()
    objs0 = [x.clone() for x in a.objs[1]]
    x = torch.zeros(16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=S):
        x.add_(1)
        st_store = hkv.status_of(a.lay.move_noalloc, hkv.HKV_OP_STORE, a.pools[1].data_ptr(), ids,
                                 a.ptrs(1, range(4)), S.cuda_stream)
        st_retrieve = hkv.status_of(a.lay.move_noalloc, hkv.HKV_OP_RETRIEVE,
                                    a.pools[1].data_ptr(), ids, a.ptrs(1, range(4)),
                                    S.cuda_stream)
    assert st_store == st_retrieve == hkv.HKV_E_CAPTURE
    assert "not in the static scratch" in hkv.hkv_last_error()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(x.cpu(), torch.ones(16))
    assert torch.equal(a.pools[1], pool0)
    assert all(torch.equal(u, v) for u, v in zip(a.objs[1], objs0))
    # outside capture the same call takes the scratch over and runs
    a.call("store", ids, list(range(4)))


def test_noalloc_threads_share_one_layout():
    """Four host threads, each with its own stream, pool and objects, call
    the no-allocation entry point with one shared layout at the same time
    (the first calls race to put its tables into the scratch; the others
    wait for that upload).  Each thread's store and retrieve match the
    oracle."""
    import threading

    import retrieve_store_chunk_amd as hkv
    cfg = W.make_config("tiny")
    lay = hkv.Layout(cfg.desc)
    ref = oracle.Layout(cfg.desc)
    used = ref.summary["pool_bytes_used"]
    nb = ref.summary["num_blocks"]
    n = 6
    # another layout's tables in the scratch first, so the threads' first calls upload
    other = Twin(many_blocks_desc(), 2, 0x5EED0E)
    other.call("store", _ids(np.random.default_rng(1), 2, other.lay.G, other.lay.k,
                             other.info["num_blocks"], distinct=True), [0, 1])
    jobs = []
    for t in range(4):
        rng = np.random.default_rng(0x5EED10 + t)
        pool_ref = W.fill_bytes(W.derive_seed(0x5EED10, t), 0, used)
        ids = _ids(rng, n, ref.G, ref.k, nb, distinct=True)
        ids2 = _ids(rng, n, ref.G, ref.k, nb, distinct=True)
        jobs.append(dict(pool=torch.from_numpy(pool_ref.copy()).to("cuda"), pool_ref=pool_ref,
                         ids=ids, ids2=ids2, stream=torch.cuda.Stream(),
                         objs=[[torch.zeros(ref.obj_bytes(o), dtype=torch.uint8, device="cuda")
                                for o in range(ref.O)] for _ in range(n)]))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(4)

    def run(j):
        try:
            ptrs = [j["objs"][c][o].data_ptr() for c in range(n) for o in range(ref.O)]
            start.wait()
            for _ in range(3):
                lay.move_noalloc(hkv.HKV_OP_STORE, j["pool"].data_ptr(), j["ids"], ptrs,
                                 j["stream"].cuda_stream)
                lay.move_noalloc(hkv.HKV_OP_RETRIEVE, j["pool"].data_ptr(), j["ids2"], ptrs,
                                 j["stream"].cuda_stream)
            j["stream"].synchronize()
        except Exception as e:  # reported after the join
            errors.append(e)

    threads = [threading.Thread(target=run, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for t, j in enumerate(jobs):
        objs_ref = [[np.zeros(ref.obj_bytes(o), np.uint8) for o in range(ref.O)]
                    for _ in range(n)]
        for _ in range(3):
            ref.store(j["pool_ref"], j["ids"], objs_ref)
            ref.retrieve(j["pool_ref"], j["ids2"], objs_ref)
        assert np.array_equal(j["pool"].cpu().numpy(), j["pool_ref"]), f"thread {t}: pool"
        for c in range(n):
            for o in range(ref.O):
                assert np.array_equal(j["objs"][c][o].cpu().numpy(), objs_ref[c][o]), \
                    f"thread {t}: object {c}/{o}"


def big_table_desc():
    # Kimi-Linear TP=1 shapes in a pool of eight blocks: tables of about 117
    # KB (14,317 work items per chunk), so some 35 such layouts fill the
    # 4 MiB scratch.
    desc = dict(W.make_config("kl_tp1").desc)
    import retrieve_store_chunk_amd as hkv
    stride = hkv.Layout(desc).info["block_stride"]
    desc["pool_bytes"] = 8 * stride
    return desc


def _store_and_retrieve(t, rng):
    nb = t.info["num_blocks"]
    t.call("store", _ids(rng, 1, t.lay.G, t.lay.k, nb, distinct=True), [0])
    t.call("retrieve", _ids(rng, 1, t.lay.G, t.lay.k, nb, distinct=True), [0])


def test_noalloc_two_layouts_in_one_graph():
    """Two layouts, both in the scratch after one eager call each, captured
    together into one HIP graph.  Two replays against the same calls made
    eagerly through the workspace entry points on the twin buffers."""
    import retrieve_store_chunk_amd as hkv
    a = Twin(W.make_config("tiny").desc, 4, 0x5EED30)
    b = Twin(many_blocks_desc(), 4, 0x5EED31)
    rng = np.random.default_rng(0x5EED32)
    calls = []
    for t in (a, b):
        nb = t.info["num_blocks"]
        t.call("store", _ids(rng, 4, t.lay.G, t.lay.k, nb, distinct=False), list(range(4)))
        calls.append((t, "store", _ids(rng, 4, t.lay.G, t.lay.k, nb, distinct=False)))
        calls.append((t, "retrieve", _ids(rng, 3, t.lay.G, t.lay.k, nb, distinct=True)))
    S = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=S):
        for t, op, ids in calls:
            code = hkv.HKV_OP_STORE if op == "store" else hkv.HKV_OP_RETRIEVE
            n = ids.shape[0]
            t.lay.move_noalloc(code, t.pools[1].data_ptr(), ids, t.ptrs(1, range(n)),
                               S.cuda_stream)
    for rep in range(2):
        graph.replay()
        for t, op, ids in calls:
            n = ids.shape[0]
            fn = t.lay.store if op == "store" else t.lay.retrieve
            fn(t.pools[0].data_ptr(), ids, t.ptrs(0, range(n)), t.ws.data_ptr(), t.ws_bytes,
               t.stream.cuda_stream)
            t.stream.synchronize()
        torch.cuda.synchronize()
        for t in (a, b):
            assert torch.equal(t.pools[0], t.pools[1]), f"replay {rep}: pools differ"
            for o in range(t.lay.O):
                assert torch.equal(t.objs[0][o], t.objs[1][o]), f"replay {rep}: objects differ"


def test_noalloc_evictions_keep_results_and_spare_captured_layouts():
    """Forty layouts of about 117 KB of tables each (more than the 4 MiB
    scratch holds), used in turn twice, so that later calls evict the least
    recently used: every call matches the workspace entry points.  A layout
    captured into a graph before them stays in the scratch, and its graph
    still replays correctly afterwards."""
    import retrieve_store_chunk_amd as hkv
    rng = np.random.default_rng(0x5EED40)
    pinned = Twin(W.make_config("tiny").desc, 4, 0x5EED41)
    nb = pinned.info["num_blocks"]
    ids_s = _ids(rng, 4, pinned.lay.G, pinned.lay.k, nb, distinct=False)
    ids_r = _ids(rng, 3, pinned.lay.G, pinned.lay.k, nb, distinct=True)
    pinned.call("store", ids_s, list(range(4)))
    S = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=S):
        pinned.lay.move_noalloc(hkv.HKV_OP_STORE, pinned.pools[1].data_ptr(), ids_s,
                                pinned.ptrs(1, range(4)), S.cuda_stream)
        pinned.lay.move_noalloc(hkv.HKV_OP_RETRIEVE, pinned.pools[1].data_ptr(), ids_r,
                                pinned.ptrs(1, range(3)), S.cuda_stream)
    desc = big_table_desc()
    twins = [Twin(desc, 1, 0x5EED50 + i) for i in range(40)]
    _log(f"[noalloc] eviction case: {len(twins)} layouts of {twins[0].info['num_blocks']} "
         f"blocks each, cycled twice")
    for cycle in range(2):
        for t in twins:
            _store_and_retrieve(t, rng)
    graph.replay()
    pinned.lay.store(pinned.pools[0].data_ptr(), ids_s, pinned.ptrs(0, range(4)),
                     pinned.ws.data_ptr(), pinned.ws_bytes, pinned.stream.cuda_stream)
    pinned.lay.retrieve(pinned.pools[0].data_ptr(), ids_r, pinned.ptrs(0, range(3)),
                        pinned.ws.data_ptr(), pinned.ws_bytes, pinned.stream.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(pinned.pools[0], pinned.pools[1]), "captured layout: pools differ"
    for o in range(pinned.lay.O):
        assert torch.equal(pinned.objs[0][o], pinned.objs[1][o]), "captured layout: objects"
    del twins
    torch.cuda.empty_cache()


def test_noalloc_trace_reports_evictions():
    """With HKV_TRACE=1 (a child process, so the setting is read fresh):
    forty layouts of about 117 KB of tables, each stored through the
    no-allocation entry point twice in turn, copy their tables in once per
    eviction, and the copies past the array's capacity report evictions."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r)\n"
        "import retrieve_store_chunk_amd as hkv\n"
        "from tests.test_zz_no_alloc import big_table_desc\n"
        "desc = big_table_desc()\n"
        "lays = [hkv.Layout(desc) for _ in range(40)]\n"
        "info = lays[0].info\n"
        "pool = torch.zeros(info['pool_bytes_used'], dtype=torch.uint8, device='cuda')\n"
        "objs = [torch.zeros(max(256, info['obj_bytes'][o]), dtype=torch.uint8, device='cuda')\n"
        "        for o in range(lays[0].O)]\n"
        "ids = np.arange(lays[0].G * lays[0].k, dtype=np.int32).reshape(1, lays[0].G, lays[0].k)\n"
        "for cycle in range(2):\n"
        "    for lay in lays:\n"
        "        lay.move_noalloc(hkv.HKV_OP_STORE, pool.data_ptr(), ids,\n"
        "                         [o.data_ptr() for o in objs])\n"
        "torch.cuda.synchronize()\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, HKV_TRACE="1"), cwd=root)
    assert r.returncode == 0, r.stderr[-3000:]
    copies = [ln for ln in r.stderr.splitlines() if "copied in at offset" in ln]
    evicting = [ln for ln in copies if not ln.endswith(" 0 layout(s) evicted")]
    # 35 fit: the first cycle copies all 40 in and evicts for the last 5; in
    # the second, each layout's range has been taken, so it is copied in again
    assert len(copies) == 80, (len(copies), r.stderr[-2000:])
    assert len(evicting) >= 45, (len(evicting), copies[:3], copies[-3:])
