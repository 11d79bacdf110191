"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default tiles, one workgroup per tile).

The pools (16-100 GiB) are too large for the oracle to copy whole, so each
wave is checked on sampled outputs the oracle's layout places one by one:
the pool and object bytes are the counter-based SplitMix64 stream, so the
expected bytes of any page or object range are computed on the host from the
seed and the oracle's placement of that page.  Also checked on samples:
store leaves the pool unchanged; retrieve leaves padding, group slack and
untargeted blocks unchanged.  Under the INT8 codec the expected object page
is the oracle's encoding of the expected pool page, and a retrieved page the
oracle's decoding of the expected object page.
"""
import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _d2h(t, lo, n):
    return t[lo:lo + n].cpu().numpy()


def _samples(rng, w, n_layers, k, count):
    """(chunk index, layer, j) samples: corners plus random ones."""
    n = len(w.chunks)
    out = {(0, 0, 0), (n - 1, n_layers - 1, k - 1)}
    cmax = int(np.unravel_index(np.argmax(w.ids), w.ids.shape)[0])
    out.add((cmax, n_layers - 1, 0))
    while len(out) < count:
        out.add((int(rng.integers(n)), int(rng.integers(n_layers)), int(rng.integers(k))))
    return sorted(out)


# Duplex workloads run their phases at once; their parity test is
# test_gpu_parity.py::test_host_duplex_parity (the sampled bookkeeping below
# follows waves in order).
FULL_SIZE = [n for n in W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES
             if not W.make_config(n).extra.get("duplex")]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_sampled(name):
    from workloads.runner import GpuWorkload
    cfg = W.make_config(name)
    print(f"[fullsize] {name}", flush=True)
    g = GpuWorkload(cfg, objects=cfg.extra.get("objects", "device"))
    ref = oracle.Layout(cfg.desc)
    assert g.info["num_blocks"] == ref.summary["num_blocks"]
    assert g.info["pool_bytes_used"] == ref.summary["pool_bytes_used"]
    Ls, k, path = ref.layers, ref.k, ref.summary["path"]
    rng = np.random.default_rng(W.derive_seed(cfg.seed, 99) % (1 << 32))
    g.init_pool()
    g.fill_objects(W.derive_seed(cfg.seed, 77))
    g.stream.synchronize()
    retrieved_since_fill = set()
    stats = {"tiles": 0, "bytes": 0, "codec": 0}

    def page_at(l, block):
        L = Ls[l]
        return L["pool_offset"] + int(block) * L["stride"], L["page_bytes"]

    N = ref.summary["block_size"]

    def valid(l, j, w, ci):
        """Bytes of page j of layer l that hold data for chunk ci of wave w."""
        L = Ls[l]
        if not L["is_mla"] or w.chunk_tokens is None:
            return L["page_bytes"]
        rows = min(N, max(0, int(w.chunk_tokens[ci]) - j * N))
        return rows * (L["page_bytes"] // N)

    def on_wave(i, w):
        nonlocal retrieved_since_fill
        if w.op == "store" and w.pool_seed is not None:
            retrieved_since_fill = set()
        fill_seed = g.current_pool_seed
        # Padding and slack keep the fill only in blocks that no earlier
        # retrieve wrote: a block another group owned before holds that
        # group's pages where this group has padding or slack.
        fresh = set(w.ids.reshape(-1).tolist()) - retrieved_since_fill
        for (ci, l, j) in _samples(rng, w, len(Ls), k, 24):
            rc = w.chunks[ci]
            L = Ls[l]
            o, grp = L["obj_group"], L["kv_group"]
            obj_n = L["obj_page_bytes"]
            obj_lo = L["obj_offset"] + j * obj_n
            codec = obj_n != L["page_bytes"]   # a KDA page in INT8 form
            bid = int(w.ids[ci, grp, j])
            if w.op == "store":
                if bid == W.NULL_BLOCK:   # a null page is zeros in the object
                    got = _d2h(g.object_view(rc, o), obj_lo, obj_n)
                    assert not got.any(), f"store wave {i} chunk {rc} layer {l} j {j}: null"
                    continue
                off, nbytes = page_at(l, bid)
                v = valid(l, j, w, ci)
                src = W.fill_bytes(g.pool_seed_of[rc], off, nbytes)
                want = ref.codec_page(src, True, l) if codec else src
                got = _d2h(g.object_view(rc, o), obj_lo, obj_n)
                if codec:
                    assert np.array_equal(got, want), f"store wave {i} chunk {rc} layer {l} j {j}"
                else:
                    assert np.array_equal(got[:v], want[:v]), \
                        f"store wave {i} chunk {rc} layer {l} j {j}"
                    assert not got[v:].any()
                # the source page is unchanged
                assert np.array_equal(_d2h(g.pool, off, nbytes), src)
            else:
                if bid == W.NULL_BLOCK:
                    continue
                v = valid(l, j, w, ci)
                if w.prefilled_objects:
                    obj_seed = W.derive_seed(W.object_seed(cfg, *rc), o)
                    want = (ref.codec_page(W.fill_bytes(obj_seed, obj_lo, obj_n), False, l)
                            if codec else W.fill_bytes(obj_seed, obj_lo, v))
                else:
                    soff, _ = page_at(l, g.store_ids[rc][grp, j])
                    want = W.fill_bytes(g.pool_seed_of[rc], soff, v)
                    if codec:
                        want = ref.codec_page(ref.codec_page(want, True, l), False, l)
                off, nbytes = page_at(l, bid)
                got = _d2h(g.pool, off, v)
                assert np.array_equal(got, want), f"retrieve wave {i} chunk {rc} layer {l} j {j}"
                # rows past a partial chunk's last token are not written
                if v < nbytes and bid in fresh:
                    assert np.array_equal(_d2h(g.pool, off + v, nbytes - v),
                                          W.fill_bytes(fill_seed, off + v, nbytes - v))
                # padding (path A) / slack (path B) after the page is untouched
                if path == 0 and L["reserved_bytes"] > nbytes and \
                        int(w.ids[ci, grp, j]) in fresh:
                    pad_lo, pad_n = off + nbytes, L["reserved_bytes"] - nbytes
                    assert np.array_equal(_d2h(g.pool, pad_lo, pad_n),
                                          W.fill_bytes(fill_seed, pad_lo, pad_n))
            stats["tiles"] += 1
            stats["bytes"] += L["page_bytes"]
            stats["codec"] += int(codec)
        if path == 1 and w.op == "retrieve":
            # group slack [group total, block stride) of targeted blocks
            totals = {}
            for L in Ls:
                totals[L["kv_group"]] = totals.get(L["kv_group"], 0) + L["page_bytes"]
            stride = ref.summary["block_stride"]
            for ci in {0, len(w.chunks) - 1}:
                for grp, tot in totals.items():
                    b = int(w.ids[ci, grp, 0])
                    if tot < stride and b in fresh and b != W.NULL_BLOCK:
                        lo = b * stride + tot
                        assert np.array_equal(_d2h(g.pool, lo, stride - tot),
                                              W.fill_bytes(fill_seed, lo, stride - tot))
        if w.op == "retrieve":
            retrieved_since_fill |= set(w.ids.reshape(-1).tolist()) - {W.NULL_BLOCK}
        # blocks no retrieve has written since the last fill still hold the fill
        free = [b for b in range(g.info["num_blocks"]) if b not in retrieved_since_fill]
        for b in rng.choice(free, size=min(4, len(free)), replace=False):
            off, nbytes = page_at(int(rng.integers(len(Ls))), b)
            assert np.array_equal(_d2h(g.pool, off, nbytes), W.fill_bytes(fill_seed, off, nbytes))

    g.run_all(on_wave=on_wave)
    g.stream.synchronize()
    print(f"[fullsize] {name}: {len(g.waves)} waves, {stats['tiles']} sampled pages "
          f"({stats['bytes'] / 1e6:.1f} MB, {stats['codec']} in INT8 form) match", flush=True)
    del g
    torch.cuda.empty_cache()
