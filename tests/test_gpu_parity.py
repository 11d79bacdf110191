"""GPU parity: the HIP library against the CPU oracle, byte for byte.

Every case runs the same seeded waves on both sides and compares the whole
pool after every wave and every object at the end.  Inputs are generated on
the host (workloads.fill_bytes) and copied to the device, so neither side's
inputs come from the other.
"""
import os

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


def run_parity(cfg, tile_bytes=0, max_workgroups=0, pool_fill=None, objects="device",
               retrieve_engine=None):
    from workloads.runner import GpuWorkload
    _log(f"[parity] {cfg.name} tile={tile_bytes} max_wg={max_workgroups} objects={objects} "
         f"retrieve={retrieve_engine}")
    g = GpuWorkload(cfg, tile_bytes=tile_bytes, max_workgroups=max_workgroups, objects=objects,
                    retrieve_engine=retrieve_engine)
    ref = oracle.Layout(cfg.desc)
    for key, okey in (("num_blocks", "num_blocks"), ("pool_bytes_used", "pool_bytes_used"),
                      ("n_kv_groups", "n_kv_groups"), ("blocks_per_chunk", "blocks_per_chunk")):
        assert g.info[key] == ref.summary[okey]
    used = ref.summary["pool_bytes_used"]
    O = ref.O

    def upload_pool(seed):
        host = pool_fill(used, seed) if pool_fill else W.fill_bytes(seed, 0, used)
        g.pool[:used].copy_(torch.from_numpy(host))
        torch.cuda.synchronize()
        return host

    pool_ref = upload_pool(W.initial_pool_seed(cfg))
    objs_ref = {}
    for rc in g.slot_of:
        objs_ref[rc] = []
        for o in range(O):
            a = W.fill_bytes(W.derive_seed(W.object_seed(cfg, *rc), o), 0, ref.obj_bytes(o))
            objs_ref[rc].append(a)
            g.object_view(rc, o).copy_(torch.from_numpy(a))
    torch.cuda.synchronize()
    for i, w in enumerate(g.waves):
        if w.op == "store" and w.pool_seed is not None:
            pool_ref = upload_pool(w.pool_seed)
        g.run_wave(w)
        g.stream.synchronize()
        objs = [objs_ref[rc] for rc in w.chunks]
        (ref.store if w.op == "store" else ref.retrieve)(pool_ref, w.ids, objs,
                                                         chunk_tokens=w.chunk_tokens)
        got = g.host_pool()
        assert np.array_equal(got, pool_ref), f"pool differs after wave {i} ({w.op})"
    for rc in g.slot_of:
        for o in range(O):
            got = g.host_object(rc, o)
            assert np.array_equal(got, objs_ref[rc][o]), f"object {rc}/{o} differs"
    n_waves = len(g.waves)
    del g
    torch.cuda.empty_cache()
    return n_waves


@pytest.mark.parametrize("name", W.CONFIG_NAMES + ("k3_tp8_holes", "kl_tp1_tails"))
def test_workload_parity_small(name):
    """The five workloads with their real page shapes, smaller pools and
    fewer requests: several waves, several tiles per page, ragged last tiles."""
    n = run_parity(W.make_small_config(name))
    assert n >= 2


@pytest.mark.parametrize("tile,max_wg", [(4096, 0), (8192, 7), (1 << 20, 1), (1 << 30, 3),
                                         (0, 13)])
def test_results_do_not_depend_on_tuning(tile, max_wg):
    run_parity(W.make_config("tiny"), tile_bytes=tile, max_workgroups=max_wg)
    run_parity(W.make_small_config("k3_tp8"), tile_bytes=tile, max_workgroups=max_wg)


def pathological(nbytes, seed):
    """bf16 / fp8 NaNs with payloads, infinities, -0, denormals, mixed with
    random bytes: a copy through float registers would change some."""
    pats = np.array([0x7FC1, 0xFFFF, 0x7F81, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80,
                     0x7F7F, 0xFFFE], dtype="<u2").view(np.uint8)
    out = W.fill_bytes(seed, 0, nbytes)
    reps = np.resize(pats, nbytes // 2 * 2)
    out[: reps.size: 2] = reps[::2]
    out[1: reps.size: 2] = np.where(np.arange(reps.size // 2) % 3 == 0,
                                    out[1: reps.size: 2], reps[1::2])
    return out


def test_pathological_bit_patterns():
    run_parity(W.make_config("tiny"), pool_fill=pathological)
    run_parity(W.make_small_config("k3_tp8"), pool_fill=pathological)


def mini_config(name, is_mla, path, sep=1, grouping=None, chunk_min=1, conv_dim=4,
                mla_width=8, mla_bytes=1, heads=1, head_dim=4, blocks=12, requests=(2, 1, 3),
                retrieve_first=None, codec=0):
    """A small layout with a given shape; the pool holds `blocks` blocks."""
    desc = W._desc(is_mla, heads, head_dim, conv_dim, mla_bytes, path, 1 << 30,
                   chunk_min=chunk_min, kv_group_of_layer=grouping, separate=sep,
                   mla_width=mla_width, kda_codec=codec)
    probe = oracle.Layout(desc).summary
    per_block = probe["pool_bytes_used"] // probe["num_blocks"]
    desc["pool_bytes"] = blocks * per_block + 5
    req = list(requests)
    store = W._all_chunks(req)
    retr = W._all_chunks(req, first=retrieve_first)
    return W.Config(name, name, desc, req, [W.Phase("store", store), W.Phase("retrieve", retr)],
                    seed=W.derive_seed(len(name), sum(is_mla), path))


EDGE = [
    # page sizes that are not 16-byte multiples (byte path) and odd offsets
    mini_config("odd_pages_A", [0, 0, 1], 0, conv_dim=5),
    mini_config("odd_pages_B", [0, 1, 0, 1], 1, conv_dim=5, mla_width=9),
    # several blocks per chunk
    mini_config("k3_blocks", [0, 1, 0], 0, chunk_min=40, blocks=30),
    # one object holding every layer; one group holding every layer
    mini_config("merged_objects", [0, 0, 0, 1], 1, sep=0),
    mini_config("one_group", [0, 1, 1, 0], 1, grouping=[0, 0, 0, 0], blocks=8),
    mini_config("group_per_layer", [1, 0, 1], 0, grouping=[2, 0, 1], blocks=12,
                requests=(1, 1, 1, 1)),
    # a single layer, only KDA, only MLA
    mini_config("single_mla", [1], 0, blocks=5, requests=(2, 3)),
    mini_config("only_kda", [0, 0, 0], 1, blocks=9),
    mini_config("only_mla", [1, 1], 1, blocks=6, requests=(3, 3)),
    # pages of several tiles (4096-byte tiles) with a ragged end
    mini_config("multi_tile", [0, 0, 1], 1, heads=3, head_dim=40, conv_dim=104, mla_width=320,
                mla_bytes=2, blocks=10),
    # the whole pool addressed: every id up to num_blocks - 1 is used
    mini_config("full_pool", [0, 0, 0, 1], 0, blocks=8, requests=(1, 1)),
    # twenty blocks per chunk (a 320-token minimum at N = 16)
    mini_config("k20_blocks", [0, 1], 1, chunk_min=320, blocks=256),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_edge_layouts(cfg):
    run_parity(cfg)
    run_parity(cfg, tile_bytes=4096, max_workgroups=3)


def holes_and_tails(cfg, every, tail):
    """The same layout with KDA snapshots every `every` blocks and a partial
    last chunk of `tail` tokens in every request."""
    import copy
    cfg = copy.deepcopy(cfg)
    tails = {(r, n - 1): tail for r, n in enumerate(cfg.requests)}
    cfg.phases = [W.Phase(ph.op, ph.chunks, ph.prefilled_objects, every, tails)
                  for ph in cfg.phases]
    cfg.name += f"_every{every}_tail{tail}"
    return cfg


def varied_tails(cfg, tails, every=1):
    """The layout with one request per entry of `tails`, each of two chunks
    whose second holds that many tokens: the chunks of a retrieve fall into
    len(set(tails)) + 1 classes."""
    import copy
    cfg = copy.deepcopy(cfg)
    cfg.requests = [2] * len(tails)
    chunks = W._all_chunks(cfg.requests)
    tt = {(r, 1): t for r, t in enumerate(tails)}
    cfg.phases = [W.Phase("store", chunks, False, every, tt),
                  W.Phase("retrieve", chunks, False, every, tt)]
    cfg.name += f"_tails{len(set(tails))}"
    return cfg


@pytest.mark.parametrize("cfg", [holes_and_tails(EDGE[0], 2, 5), holes_and_tails(EDGE[1], 1, 1),
                                 holes_and_tails(EDGE[2], 3, 33),
                                 holes_and_tails(EDGE[9], 2, 17),
                                 holes_and_tails(EDGE[2], 1, 0),
                                 holes_and_tails(EDGE[11], 4, 150)],
                         ids=lambda c: c.name)
def test_edge_layouts_with_holes_and_tails(cfg):
    """Null ids and partial chunks on odd page sizes (byte path), several
    blocks per chunk and multi-tile pages (4 KiB tiles); a tail of 0 tokens
    makes a chunk whose ids are all null."""
    run_parity(cfg)
    run_parity(cfg, tile_bytes=4096, max_workgroups=5)


@pytest.mark.parametrize("name", ["tiny", "kl_tp1_host", "k3_tp8", "long_ctx"])
def test_host_object_parity(name):
    """Chunk objects in pinned host memory (the GPU reads and writes them over
    the host link): the same bytes as the oracle."""
    run_parity(W.make_small_config(name), objects="host")


@pytest.mark.parametrize("cfg", [EDGE[0], EDGE[2]], ids=lambda c: c.name)
def test_host_object_parity_edge_layouts(cfg):
    run_parity(cfg, objects="host")


def test_empty_batch_is_a_noop():
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    g = GpuWorkload(W.make_config("tiny"))
    g.init_pool()
    before = g.host_pool().copy()
    empty = np.zeros((0, g.layout.G, g.layout.k), np.int32)
    hkv.hkv_store_chunks(g.layout.handle, g.pool.data_ptr(), empty, [], g.ws.data_ptr(),
                         g.ws_bytes, g.stream.cuda_stream)
    hkv.hkv_retrieve_chunks(g.layout.handle, g.pool.data_ptr(), empty, [], g.ws.data_ptr(),
                            g.ws_bytes, g.stream.cuda_stream)
    assert np.array_equal(g.host_pool(), before)


def test_error_paths_enqueue_nothing():
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    g = GpuWorkload(W.make_config("tiny"))
    g.init_pool()
    g.fill_objects(5)
    g.stream.synchronize()
    pool0 = g.host_pool().copy()
    w = g.waves[0]
    ptrs = g.object_ptrs(w.chunks)
    h, s = g.layout.handle, g.stream.cuda_stream
    P, WS = g.pool.data_ptr(), g.ws.data_ptr()
    nb = g.info["num_blocks"]
    bad = w.ids.copy()
    bad[-1, -1, -1] = nb
    cases = [
        (hkv.hkv_retrieve_chunks, (h, P, bad, ptrs, WS, g.ws_bytes, s), hkv.HKV_E_RANGE),
        (hkv.hkv_store_chunks, (h, P, bad, ptrs, WS, g.ws_bytes, s), hkv.HKV_E_RANGE),
        (hkv.hkv_retrieve_chunks, (h, P + 8, w.ids, ptrs, WS, g.ws_bytes, s), hkv.HKV_E_ALIGN),
        (hkv.hkv_retrieve_chunks, (h, P, w.ids, ptrs, WS, 16, s), hkv.HKV_E_WORKSPACE),
        (hkv.hkv_store_chunks, (h, P, w.ids, [ptrs[0]] * len(ptrs), WS, g.ws_bytes, s),
         hkv.HKV_E_ALIAS),
    ]
    if len(w.chunks) > 1:
        dup = w.ids.copy()
        dup[1, 0, 0] = dup[0, 0, 0]
        cases.append((hkv.hkv_retrieve_chunks, (h, P, dup, ptrs, WS, g.ws_bytes, s),
                      hkv.HKV_E_ALIAS))
    for fn, args, want in cases:
        assert hkv.status_of(fn, *args) == want
    g.stream.synchronize()
    assert np.array_equal(g.host_pool(), pool0)


def test_gpu_fill_matches_host_generator():
    t = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for seed, start, n in [(1, 0, 1 << 20), (0x48B0003, 4096, 12345), (7, 8, 7)]:
        W.gpu_fill(t.data_ptr(), n, seed, start)
        torch.cuda.synchronize()
        assert np.array_equal(t[:n].cpu().numpy(), W.fill_bytes(seed, start, n))


def test_objects_move_between_pool_layouts_with_equal_fingerprints():
    """Equal fingerprints mean interchangeable objects: chunks stored from a
    path B pool are retrieved into a path A pool of the same model, matching
    the oracle byte for byte, and storing them again from path A gives the
    same objects."""
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    cfg_b = W.make_small_config("kl_tp1")
    cfg_a = W.make_small_config("kl_tp1")
    cfg_a.desc = dict(cfg_a.desc, path=0)
    gb, ga = GpuWorkload(cfg_b), GpuWorkload(cfg_a)
    assert gb.layout.fingerprint() == ga.layout.fingerprint()
    ref_a = oracle.Layout(cfg_a.desc)
    gb.init_pool()
    gb.fill_objects(1)
    store = gb.waves[0]
    gb.run_wave(store)
    gb.stream.synchronize()
    objs_b = [[gb.host_object(rc, o) for o in range(ref_a.O)] for rc in store.chunks]
    # retrieve B's objects into A's pool at A's fresh ids
    ga.init_pool()
    ga.stream.synchronize()
    used = ref_a.summary["pool_bytes_used"]
    pool_a = ga.host_pool().copy()
    ids_a = W.permutation(W.derive_seed(cfg_a.seed, 4242), ref_a.summary["num_blocks"])
    ids_a = ids_a[: len(store.chunks) * ref_a.G * ref_a.k].reshape(len(store.chunks), ref_a.G,
                                                                  ref_a.k).copy()
    hkv.hkv_retrieve_chunks(ga.layout.handle, ga.pool.data_ptr(), ids_a,
                            gb.object_ptrs(store.chunks), ga.ws.data_ptr(), ga.ws_bytes,
                            ga.stream.cuda_stream)
    ref_a.retrieve(pool_a, ids_a, objs_b)
    assert np.array_equal(ga.host_pool()[:used], pool_a)
    # storing from path A reproduces the objects stored from path B
    hkv.hkv_store_chunks(ga.layout.handle, ga.pool.data_ptr(), ids_a,
                         ga.object_ptrs(store.chunks), ga.ws.data_ptr(), ga.ws_bytes,
                         ga.stream.cuda_stream)
    for n, rc in enumerate(store.chunks):
        for o in range(ref_a.O):
            assert np.array_equal(ga.host_object(rc, o), objs_b[n][o])


# ------------------------------------------------------------ INT8 codec
def with_codec(cfg):
    import copy
    cfg = copy.deepcopy(cfg)
    cfg.desc = dict(cfg.desc, kda_codec=1)
    cfg.name += "_int8"
    return cfg


@pytest.mark.parametrize("name", ["kl_tp1_int8", "tiny", "kl_tp2", "k3_tp8", "long_ctx",
                                  "k3_tp8_holes", "kl_tp1_tails"])
def test_codec_workload_parity_small(name):
    """Workload shapes under the INT8 codec.  The pool and objects are random
    bytes, so the fp32 states span every bit pattern (NaNs with payloads,
    infinities, denormals, every exponent) and the long-context retrieve
    decodes objects no encoder wrote."""
    cfg = W.make_small_config(name)
    run_parity(cfg if cfg.desc.get("kda_codec") else with_codec(cfg))


CODEC_EDGE = [
    # d = 16 (4 lanes a row), conv part of 3 x 16 bytes
    mini_config("codec_d16", [0, 0, 1], 0, heads=1, head_dim=16, conv_dim=8, codec=1),
    # no conv part, odd MLA pages (byte path beside the codec)
    mini_config("codec_d32_noconv", [0, 1, 0, 1], 1, heads=2, head_dim=32, conv_dim=0,
                mla_width=9, codec=1),
    # d = 64, two blocks per chunk, conv part of several tiles
    mini_config("codec_d64_k2", [0, 1, 0], 0, heads=3, head_dim=64, conv_dim=104,
                mla_width=1024, mla_bytes=2, chunk_min=40, blocks=30, codec=1),
    # d = 256 (16 lanes a row, 4 vectors a lane), one object for every layer
    mini_config("codec_d256_merged", [0, 0, 1], 1, sep=0, heads=1, head_dim=256, conv_dim=8,
                mla_width=512, mla_bytes=2, blocks=16, codec=1),
    mini_config("codec_only_kda", [0, 0, 0], 1, heads=2, head_dim=16, conv_dim=8, blocks=9,
                codec=1),
]


def codec_rows(rng, n, d):
    """n rows of d fp32 values from eight recipes: Gaussian at random scales,
    exact ties (largest |x| = 127 * 2^e, the rest (m + 1/2) * 2^e), exact
    power-of-two lattices, denormals, zero rows, NaN / inf sprinkled into a
    row, rows with nothing finite, and values near the fp32 maximum."""
    kind = rng.integers(0, 8, n)
    e = np.exp2(rng.integers(-30, 30, (n, 1))).astype(np.float32)
    x = (rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-3, 3, (n, 1))).astype(np.float32)
    ties = ((rng.integers(-127, 127, (n, d)) + 0.5) * e).astype(np.float32)
    ties[:, 0] = 127 * e[:, 0] * np.where(rng.random(n) < 0.5, -1, 1)
    lattice = (rng.integers(-127, 128, (n, d)) * e).astype(np.float32)
    denorm = (rng.standard_normal((n, d)) * 1e-39).astype(np.float32)
    zero = np.where(rng.random((n, d)) < 0.5, 0.0, -0.0).astype(np.float32)
    sprinkled = x.copy()
    hit = rng.random((n, d)) < 0.1
    sprinkled[hit] = rng.choice(np.array([np.nan, np.inf, -np.inf], np.float32), hit.sum())
    nothing = rng.choice(np.array([np.nan, np.inf, -np.inf], np.float32), (n, d))
    huge = (rng.uniform(-1, 1, (n, d)) * np.finfo(np.float32).max).astype(np.float32)
    out = np.choose(kind[:, None], [x, ties, lattice, denorm, zero, sprinkled, nothing, huge])
    return out.astype(np.float32)


def codec_fill(desc):
    """A pool fill: random bytes, with every KDA page's recurrent rows (in
    every block) drawn from codec_rows."""
    ref = oracle.Layout(desc)
    d = desc["kda_head_dim"]
    rows = desc["kda_heads"] * d
    conv = desc["conv_dim"] * (desc["conv_kernel"] - 1) * desc["conv_bytes"]

    def fill(nbytes, seed):
        out = W.fill_bytes(seed, 0, nbytes)
        rng = np.random.default_rng(seed % (1 << 32))
        for L in ref.layers:
            if L["is_mla"]:
                continue
            for b in range(ref.summary["num_blocks"]):
                lo = L["pool_offset"] + b * L["stride"] + conv
                out[lo: lo + rows * d * 4] = codec_rows(rng, rows, d).view(np.uint8).ravel()
        return out
    return fill


@pytest.mark.parametrize("cfg", [with_codec(W.make_config("tiny"))] + CODEC_EDGE,
                         ids=lambda c: c.name)
def test_codec_value_recipes(cfg):
    """Rows built to hit every branch of the quantiser: bit-exact codes,
    scales and decoded states against the oracle."""
    run_parity(cfg, pool_fill=codec_fill(cfg.desc))


@pytest.mark.parametrize("cfg", CODEC_EDGE, ids=lambda c: c.name)
@pytest.mark.parametrize("tile,max_wg", [(0, 0), (8192, 7), (1 << 20, 1)])
def test_codec_edge_layouts_and_tuning(cfg, tile, max_wg):
    """Rows per codec item follow the tile size; results do not."""
    run_parity(cfg, tile_bytes=tile, max_workgroups=max_wg)


@pytest.mark.parametrize("cfg", [holes_and_tails(CODEC_EDGE[0], 2, 5),
                                 holes_and_tails(CODEC_EDGE[2], 3, 33),
                                 holes_and_tails(CODEC_EDGE[3], 1, 100),
                                 holes_and_tails(CODEC_EDGE[2], 2, 0)],
                         ids=lambda c: c.name)
def test_codec_with_holes_and_tails(cfg):
    """Null KDA pages (codes and scales zeroed on store, nothing written on
    retrieve) beside partial MLA chunks."""
    run_parity(cfg, pool_fill=codec_fill(cfg.desc))
    run_parity(cfg, tile_bytes=4096, max_workgroups=5)


def test_codec_host_objects():
    cfg = W.make_small_config("kl_tp1_int8_host")
    assert cfg.extra["objects"] == "host" and cfg.desc["kda_codec"] == 1
    run_parity(cfg, objects="host")


@pytest.mark.parametrize("first_on_host", [True, False], ids=["host_first", "device_first"])
@pytest.mark.parametrize("cfg", [CODEC_EDGE[0], CODEC_EDGE[2], CODEC_EDGE[3]], ids=lambda c: c.name)
def test_codec_store_with_objects_in_both_memories(cfg, first_on_host):
    """An INT8 store whose objects are split between pinned host memory and
    device memory (every other chunk): the first object picks the gather
    form, and either form writes the oracle's bytes into both kinds of
    memory."""
    import retrieve_store_chunk_amd as hkv
    ref = oracle.Layout(cfg.desc)
    lay = hkv.Layout(cfg.desc)
    used = ref.summary["pool_bytes_used"]
    pool_ref = codec_fill(cfg.desc)(used, W.derive_seed(cfg.seed, 91))
    pool = torch.from_numpy(pool_ref).to("cuda")
    n = 6
    rng = np.random.default_rng(0x5EED20)
    # (a store may read one block for several chunks)
    ids = rng.integers(0, ref.summary["num_blocks"], size=(n, ref.G, ref.k)).astype(np.int32)
    objs = []
    for c in range(n):
        on_host = (c % 2 == 0) == first_on_host
        objs.append([torch.full((ref.obj_bytes(o),), 0xA5, dtype=torch.uint8,
                                pin_memory=True) if on_host else
                     torch.full((ref.obj_bytes(o),), 0xA5, dtype=torch.uint8, device="cuda")
                     for o in range(ref.O)])
    objs_ref = [[np.full(ref.obj_bytes(o), 0xA5, np.uint8) for o in range(ref.O)]
                for _ in range(n)]
    ptrs = [objs[c][o].data_ptr() for c in range(n) for o in range(ref.O)]
    ws_bytes = lay.workspace_size(n)
    ws = torch.empty(max(256, ws_bytes), dtype=torch.uint8, device="cuda")
    ref.store(pool_ref, ids, objs_ref)
    for entry in ("workspace", "noalloc"):
        for row in objs:
            for t in row:
                t.fill_(0xA5)
        torch.cuda.synchronize()
        if entry == "workspace":
            lay.store(pool.data_ptr(), ids, ptrs, ws.data_ptr(), ws_bytes, 0)
        else:
            lay.move_noalloc(hkv.HKV_OP_STORE, pool.data_ptr(), ids, ptrs, 0)
        torch.cuda.synchronize()
        for c in range(n):
            for o in range(ref.O):
                assert np.array_equal(objs[c][o].cpu().numpy(), objs_ref[c][o]), \
                    f"{entry}: object {c}/{o}"


@pytest.mark.parametrize("cfg", CODEC_EDGE + [holes_and_tails(CODEC_EDGE[2], 3, 33)],
                         ids=lambda c: c.name)
def test_codec_edge_layouts_host_objects(cfg):
    """Stores into objects in pinned host memory write each row's codes with
    line-wide stores after a lane exchange: every head_dim (1, 2 or 4 code
    words a lane), null pages and partial chunks, against the oracle."""
    run_parity(cfg, objects="host", pool_fill=codec_fill(cfg.desc))


@pytest.mark.parametrize("cfg", [varied_tails(mini_config("varied", [0, 1, 0, 1], 1, chunk_min=40,
                                                           blocks=80), [3, 17, 3, 40, 17, 0]),
                                 varied_tails(mini_config("varied", [0, 1, 0, 1], 1, chunk_min=40,
                                                          blocks=240), list(range(1, 40, 3))),
                                 varied_tails(CODEC_EDGE[2], [5, 33, 5, 0], every=2)],
                         ids=lambda c: c.name)
def test_retrieve_classes_and_plain_fallback(cfg):
    """A retrieve whose chunks fall into a few classes (same null ids, same
    token count) launches once per class over only the work items that
    write something; with more than 8 classes it makes one launch over every
    item.  Both must match the oracle byte for byte."""
    run_parity(cfg)
    run_parity(cfg, tile_bytes=4096, max_workgroups=5)


def call_size_config(n, tails):
    """n one-chunk requests of a two-group layout, all in one call: 3 words of
    per-call tables a chunk (ids, two object addresses), plus half a word
    with token counts, against 384 words of kernel arguments."""
    import copy
    cfg = mini_config(f"calls{n}", [0, 1], 1, blocks=2 * n + 8, requests=(1,) * n)
    cfg = copy.deepcopy(cfg)
    chunks = W._all_chunks(cfg.requests)
    tt = {(r, 0): 1 + r % 15 for r in range(n)} if tails else {}
    cfg.phases = [W.Phase("store", chunks, False, 1, tt), W.Phase("retrieve", chunks, False, 1, tt)]
    cfg.name += "_tails" if tails else ""
    return cfg


@pytest.mark.parametrize("n,tails", [(128, False), (129, False), (109, True), (110, True)])
def test_calls_at_the_kernel_argument_limit(n, tails):
    """A call whose per-call tables fit in the kernel arguments (128 chunks
    here, 109 with token counts) is one launch; one chunk more goes through
    the workspace.  Both sides of the limit match the oracle."""
    cfg = call_size_config(n, tails)
    ref = oracle.Layout(cfg.desc)
    assert (ref.G, ref.k, ref.O) == (2, 1, 2)
    run_parity(cfg)


def random_layout_cases(n_cases=100, seed=2026):
    """Seeded random small layouts: layer pattern, head count and head_dim,
    conv and MLA widths and dtypes, path, object grouping, chunk minimum, the
    INT8 codec where the shape allows it, snapshot spacing, tails and tuning.
    Cases the oracle rejects are redrawn."""
    import copy
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        n_layers = int(rng.integers(1, 7))
        is_mla = [int(x) for x in rng.integers(0, 2, n_layers)]
        heads = int(rng.integers(1, 4))
        head_dim = int(rng.choice([4, 8, 16, 32, 64]))
        conv_dim = int(rng.choice([0, 4, 5, 8, 24]))
        mla_width = int(rng.choice([8, 9, 64, 576]))
        mla_bytes = int(rng.choice([1, 2]))
        codec = int(head_dim >= 16 and (conv_dim * 3 * 2) % 16 == 0 and rng.random() < 0.5)
        desc = W._desc(is_mla, heads, head_dim, conv_dim, mla_bytes, int(rng.integers(0, 2)),
                       1 << 30, chunk_min=int(rng.integers(1, 60)),
                       separate=int(rng.integers(0, 2)), mla_width=mla_width, kda_codec=codec)
        try:
            probe = oracle.Layout(desc)
        except oracle.OracleError:
            continue
        s = probe.summary
        per_block = s["pool_bytes_used"] // s["num_blocks"]
        requests = [int(x) for x in rng.integers(1, 4, int(rng.integers(1, 5)))]
        ids_needed = sum(requests) * probe.G * probe.k
        desc["pool_bytes"] = (ids_needed + int(rng.integers(0, 6))) * per_block + 7
        every = int(rng.choice([1, 1, 2, 3]))
        tails = {}
        if rng.random() < 0.5:
            tails = {(r, n - 1): int(rng.integers(0, s["chunk_tokens"] + 1))
                     for r, n in enumerate(requests)}
        chunks = W._all_chunks(requests)
        name = f"rand{len(cases)}"
        cfg = W.Config(name, name, desc, requests,
                       [W.Phase("store", chunks, False, every, tails),
                        W.Phase("retrieve", chunks, False, every, tails)],
                       seed=W.derive_seed(seed, len(cases)))
        tile = int(rng.choice([0, 4096, 8192, 1 << 20]))
        max_wg = int(rng.choice([0, 0, 1, 5, 64]))
        cases.append((cfg, tile, max_wg))
    return cases


@pytest.mark.parametrize("case", random_layout_cases(), ids=lambda c: c[0].name)
def test_random_layouts(case):
    """Random small layouts, byte for byte against the oracle."""
    cfg, tile, max_wg = case
    run_parity(cfg, tile_bytes=tile, max_workgroups=max_wg)


def test_host_duplex_parity():
    """A store and a retrieve at the same time on two streams, objects in
    pinned host memory (the host link carries both directions at once).  The
    two touch different blocks and objects, so the result is the oracle's
    retrieve and store applied one after the other."""
    from workloads.runner import GpuWorkload
    cfg = W.make_small_config("kl_tp1_host_duplex")
    g = GpuWorkload(cfg, objects="host")
    ref = oracle.Layout(cfg.desc)
    used = ref.summary["pool_bytes_used"]
    g.init_pool()
    g.fill_objects(W.derive_seed(cfg.seed, 77))
    g.synchronize()
    torch.cuda.synchronize()
    g.run_all()
    torch.cuda.synchronize()
    # the oracle: the same fills, then the waves in turn
    ret = [w for w in g.waves if w.op == "retrieve"]
    sto = [w for w in g.waves if w.op == "store"]
    assert len(sto) == 1 and ret
    seed = sto[0].pool_seed if sto[0].pool_seed is not None else W.initial_pool_seed(cfg)
    pool_ref = W.fill_bytes(seed, 0, used)
    objs_ref = {}
    for rc in g.slot_of:
        objs_ref[rc] = [W.fill_bytes(W.derive_seed(W.derive_seed(cfg.seed, 77), o),
                                     g.slot_of[rc] * g.obj_stride[o], ref.obj_bytes(o))
                        for o in range(ref.O)]
    for w in ret:  # prefilled objects
        for rc in w.chunks:
            objs_ref[rc] = [W.fill_bytes(W.derive_seed(W.object_seed(cfg, *rc), o), 0,
                                         ref.obj_bytes(o)) for o in range(ref.O)]
    retrieved = {int(x) for w in ret for x in w.ids.ravel()} - {W.NULL_BLOCK}
    stored = {int(x) for x in sto[0].ids.ravel()} - {W.NULL_BLOCK}
    assert not retrieved & stored
    for w in ret + sto:
        (ref.store if w.op == "store" else ref.retrieve)(
            pool_ref, w.ids, [objs_ref[rc] for rc in w.chunks], chunk_tokens=w.chunk_tokens)
    assert np.array_equal(g.host_pool(), pool_ref)
    for rc in g.slot_of:
        for o in range(ref.O):
            assert np.array_equal(g.host_object(rc, o), objs_ref[rc][o]), f"object {rc}/{o}"


DMA_CASES = ([(W.make_small_config(n), "device") for n in
              ("tiny", "kl_tp2", "k3_tp8", "long_ctx", "k3_tp8_holes", "kl_tp1_tails")] +
             [(W.make_small_config("kl_tp1_host"), "host"), (W.make_config("tiny"), "host")] +
             [(c, "device") for c in (EDGE[0], EDGE[1], EDGE[2], EDGE[3],
                                      holes_and_tails(EDGE[2], 3, 33),
                                      holes_and_tails(EDGE[1], 1, 0))] +
             [(c, "device") for c, _, _ in random_layout_cases() if not c.desc["kda_codec"]][:20])


@pytest.mark.parametrize("case", DMA_CASES, ids=lambda c: f"{c[0].name}-{c[1]}")
def test_dma_retrieve_parity(case):
    """Retrieves by DMA copies of contiguous page runs (objects in HBM or in
    pinned host memory): the same bytes as the oracle, and as the kernels."""
    cfg, objects = case
    run_parity(cfg, objects=objects, retrieve_engine="dma")


# ------------------------------------------------------------ graph capture
GRAPH_CASES = [("tiny", "kernel"), ("kl_tp1", "kernel"), ("kl_tp1", "dma"),
               ("kl_tp1_tails", "kernel"), ("k3_tp8_holes", "kernel"),
               ("kl_tp1_int8", "kernel"), ("kl_tp1_int8_host", "kernel")]


def _first_calls(g, m):
    """The first store and the first retrieve wave, cut to m chunks each:
    (chunks, ids, chunk_tokens) per call."""
    out = []
    for op in ("store", "retrieve"):
        w = next(w for w in g.waves if w.op == op)
        tok = None if w.chunk_tokens is None else w.chunk_tokens[:m].copy()
        out.append((w.chunks[:m], w.ids[:m].copy(), tok))
    return out


@pytest.mark.parametrize("name,engine", GRAPH_CASES, ids=lambda x: str(x))
def test_graph_capture_replays_small_calls(name, engine):
    """A store and a retrieve whose tables fit in the kernel arguments are
    captured into one HIP graph.  The graph is replayed three times, with new
    pool and object bytes written eagerly before each replay, and every
    replay matches the oracle applied to that replay's inputs."""
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    cfg = W.make_config(name) if name == "tiny" else W.make_small_config(name)
    _log(f"[graph] {name} retrieve={engine}")
    g = GpuWorkload(cfg, retrieve_engine=engine, objects=cfg.extra.get("objects", "device"))
    ref = oracle.Layout(cfg.desc)
    (s_chunks, s_ids, s_tok), (r_chunks, r_ids, r_tok) = _first_calls(g, 8)
    h, P, WS, wsb, S = g.layout.handle, g.pool.data_ptr(), g.ws.data_ptr(), g.ws_bytes, g.stream
    eng = hkv.HKV_ENGINE_DMA if engine == "dma" else hkv.HKV_ENGINE_KERNEL
    # the layout's first call on the device uploads its tables: not in a capture
    g.init_pool()
    hkv.hkv_store_chunks(h, P, s_ids, g.object_ptrs(s_chunks), WS, wsb, S.cuda_stream,
                         chunk_tokens=s_tok)
    S.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=S):
        hkv.hkv_store_chunks(h, P, s_ids, g.object_ptrs(s_chunks), WS, wsb, S.cuda_stream,
                             chunk_tokens=s_tok)
        hkv.hkv_retrieve_chunks(h, P, r_ids, g.object_ptrs(r_chunks), WS, wsb, S.cuda_stream,
                                chunk_tokens=r_tok, engine=eng)
    used = ref.summary["pool_bytes_used"]
    slots = list(dict.fromkeys(list(s_chunks) + list(r_chunks)))
    for rep in range(3):
        seed = W.derive_seed(cfg.seed, 7100 + rep)
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


def test_capture_refuses_calls_it_cannot_replay():
    """Under capture, a layout's first call on the device and a call whose
    tables need the workspace return HKV_E_CAPTURE and enqueue nothing."""
    import retrieve_store_chunk_amd as hkv
    from workloads.runner import GpuWorkload
    cfg = call_size_config(129, False)
    g = GpuWorkload(cfg)
    g.init_pool()
    g.fill_objects(3)
    torch.cuda.synchronize()
    w = next(w for w in g.waves if w.op == "store")
    assert len(w.chunks) == 129
    h, P, WS, wsb, S = g.layout.handle, g.pool.data_ptr(), g.ws.data_ptr(), g.ws_bytes, g.stream
    ptrs = g.object_ptrs(w.chunks)
    pool0 = g.host_pool().copy()
    objs0 = [g.host_object(rc, o) for rc in w.chunks for o in range(g.layout.O)]
    x = torch.zeros(16, device=g.device)
    first = torch.cuda.CUDAGraph()
    with torch.cuda.graph(first, stream=S):
        x.add_(1)
        st_first = hkv.status_of(hkv.hkv_store_chunks, h, P, w.ids[:1], ptrs[:g.layout.O], WS,
                                 wsb, S.cuda_stream)
    assert st_first == hkv.HKV_E_CAPTURE
    hkv.hkv_store_chunks(h, P, w.ids[:1], ptrs[:g.layout.O], WS, wsb, S.cuda_stream)
    S.synchronize()
    objs0[:g.layout.O] = [g.host_object(w.chunks[0], o) for o in range(g.layout.O)]
    large = torch.cuda.CUDAGraph()
    with torch.cuda.graph(large, stream=S):
        x.add_(1)
        st_store = hkv.status_of(hkv.hkv_store_chunks, h, P, w.ids, ptrs, WS, wsb, S.cuda_stream)
        st_retrieve = hkv.status_of(hkv.hkv_retrieve_chunks, h, P, w.ids, ptrs, WS, wsb,
                                    S.cuda_stream)
    assert st_store == st_retrieve == hkv.HKV_E_CAPTURE
    first.replay()
    large.replay()
    torch.cuda.synchronize()
    assert torch.equal(x.cpu(), torch.full((16,), 2.0))
    assert np.array_equal(g.host_pool(), pool0)
    got = [g.host_object(rc, o) for rc in w.chunks for o in range(g.layout.O)]
    assert all(np.array_equal(a, b) for a, b in zip(got, objs0))


# ------------------------------------------------------------ threads
def test_calls_from_several_threads_at_once():
    """Four host threads call store, then retrieve, at the same moment on one
    shared layout, each on its own stream with its own workspace.  The first
    calls are the layout's first on the device (its table upload), and every
    batch is too large for the kernel arguments (its tables go through the
    shared staging ring).  Retrieve targets are disjoint across threads.
    Every object and the whole pool match the oracle."""
    import threading
    import retrieve_store_chunk_amd as hkv
    desc = W._desc([0, 0, 1, 0, 1], 1, 16, 8, 2, 1, 1 << 28, mla_width=576)
    lay, ref = hkv.Layout(desc), oracle.Layout(desc)
    G, k, O = lay.G, lay.k, lay.O
    nb, used = lay.info["num_blocks"], lay.info["pool_bytes_used"]
    n_threads, n = 4, 200
    assert (n * G * k + 1) // 2 + n * O > 384  # past the kernel-argument tables
    assert n_threads * n * G * k <= nb
    _log(f"[threads] {n_threads} x {n} chunks, G={G} k={k} O={O} blocks={nb}")
    dev = torch.device("cuda")
    pool_ref = W.fill_bytes(0x7EAD, 0, used)
    pool = torch.from_numpy(pool_ref.copy()).to(dev)
    rng = np.random.default_rng(0x7EAD)
    stride = [max(256, (lay.info["obj_bytes"][o] + 255) // 256 * 256) for o in range(O)]
    objs = [[torch.empty(n * stride[o], dtype=torch.uint8, device=dev) for o in range(O)]
            for _ in range(n_threads)]
    ptrs = [[objs[t][o].data_ptr() + c * stride[o] for c in range(n) for o in range(O)]
            for t in range(n_threads)]
    store_ids = [rng.integers(0, nb, (n, G, k)).astype(np.int32) for _ in range(n_threads)]
    perm = rng.permutation(nb)[: n_threads * n * G * k].astype(np.int32)
    retr_ids = [perm[t * n * G * k:(t + 1) * n * G * k].reshape(n, G, k).copy()
                for t in range(n_threads)]
    wsb = lay.workspace_size(n)
    ws = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(n_threads)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(n_threads)]
    torch.cuda.synchronize()
    start = threading.Barrier(n_threads)
    errors = []

    def worker(t, op):
        try:
            start.wait()
            fn, ids = (lay.store, store_ids[t]) if op == "store" else (lay.retrieve, retr_ids[t])
            fn(pool.data_ptr(), ids, ptrs[t], ws[t].data_ptr(), wsb, streams[t].cuda_stream)
            streams[t].synchronize()
        except Exception as e:  # reported after the join
            errors.append((t, op, repr(e)))

    for op in ("store", "retrieve"):
        threads = [threading.Thread(target=worker, args=(t, op)) for t in range(n_threads)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        assert not errors, errors
    torch.cuda.synchronize()
    # the oracle, one thread after another (stores read the pool before any
    # retrieve writes it; retrieve targets are disjoint)
    objs_ref = [[[np.zeros(ref.obj_bytes(o), np.uint8) for o in range(O)] for _ in range(n)]
                for _ in range(n_threads)]
    for t in range(n_threads):
        ref.store(pool_ref, store_ids[t], objs_ref[t])
    for t in range(n_threads):
        ref.retrieve(pool_ref, retr_ids[t], objs_ref[t])
    for t in range(n_threads):
        for o in range(O):
            got = objs[t][o].cpu().numpy().reshape(n, stride[o])[:, :ref.obj_bytes(o)]
            want = np.stack([objs_ref[t][c][o] for c in range(n)])
            assert np.array_equal(got, want), f"thread {t} objects {o}"
    assert np.array_equal(pool[:used].cpu().numpy(), pool_ref), "pool"


def test_trace_names_the_line_code_gather_for_host_objects(tmp_path):
    """With HKV_TRACE=1, an INT8 store into pinned host memory reports the
    line-code gather, and one into device memory does not (a child process,
    so the trace setting is read fresh)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys, torch; sys.path.insert(0, %r)\n"
        "import workloads as W\n"
        "from workloads.runner import GpuWorkload\n"
        "for objects in ('host', 'device'):\n"
        "    g = GpuWorkload(W.make_small_config('kl_tp1_int8_host'), objects=objects)\n"
        "    g.init_pool()\n"
        "    w = next(w for w in g.waves if w.op == 'store')\n"
        "    print('[objects] ' + objects, file=sys.stderr, flush=True)\n"
        "    g.run_wave(w)\n"
        "    torch.cuda.synchronize()\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, HKV_TRACE="1"), cwd=root)
    assert r.returncode == 0, r.stderr[-3000:]
    host_part, device_part = r.stderr.split("[objects] host", 1)[1].split("[objects] device", 1)
    assert "line-code gather" in host_part, host_part[-2000:]
    assert "store" in device_part and "line-code gather" not in device_part, device_part[-2000:]
