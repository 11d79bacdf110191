"""Checks every pool and object byte of a workload run against expected
bytes rebuilt from the seeded generator at the oracle's placements.

Test infrastructure shared by the full-size GPU test (expected bytes built on
the device) and a CPU test of the checker itself (built on the host, run
against the oracle).  The store/retrieve library is never called here.

- **Pool**, after every wave: the whole pool buffer against the fill of the
  last refill, overlaid, in order, by every page retrieved since then.  A
  retrieved page holds the bytes its object was stored from (the pool stream
  at the oracle's address of the stored block) or prefilled with (the
  object's stream), and zeros where the store wrote zeros (null pages, rows
  past a partial chunk's tokens).  So store leaves the pool unchanged, and a
  retrieve writes exactly its pages' valid bytes: padding, group slack and
  every other block keep their bytes.
- **Objects**, after every wave the slots it used, and at the end every
  slot, each in full including the bytes between slots: the object fill,
  then the prefilled stream, then the pages of the slot's store.  So a
  retrieve leaves objects unchanged and a store writes exactly its object.
- **INT8 codec pages** (KDA pages under the codec) cannot be rebuilt from a
  stream: in the rebuilt buffers they are taken as they are, and every
  non-null one is compared on the host against the oracle's codec of its
  expected source bytes (encode for a store, decode of the encoded object for
  a retrieve), in a pool of host threads.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads as W

ZEROS = W.ROW_ZEROS


class DeviceBuild:
    """Expected bytes built on the GPU (the generator's fill kernels)."""
    device = "cuda"
    slice_bytes = 4 << 30      # expected-pool slice built at a time
    obj_batch_bytes = 4 << 30  # expected-object bytes built at a time

    def fill(self, t, seed, byte_start):
        W.gpu_fill(t.data_ptr(), t.numel(), seed, byte_start)
        torch.cuda.synchronize()

    def fill_rows(self, t, rows):
        W.gpu_fill_rows(t, rows)

    def sync(self):
        torch.cuda.synchronize()


class HostBuild:
    """The same on the host (numpy), for checking the checker on the CPU."""
    device = "cpu"
    slice_bytes = 1 << 20
    obj_batch_bytes = 1 << 20

    def fill(self, t, seed, byte_start):
        t.numpy()[:] = W.fill_bytes(seed, byte_start, t.numel())

    def fill_rows(self, t, rows):
        a = t.numpy()
        for off, seed, word0, count in np.asarray(rows, dtype=np.uint64).reshape(-1, 4):
            n = int(count) & (ZEROS - 1)
            lo = int(off)
            if int(count) & ZEROS:
                a[lo:lo + 8 * n] = 0
            else:
                a[lo:lo + 8 * n] = W.fill_bytes(int(seed), int(word0) * 8, 8 * n)

    def sync(self):
        pass


def _rows(off, seed, word0, nbytes, zeros=False):
    """Row table entries (see workloads.gpu_fill_rows) for byte ranges."""
    off = np.asarray(off, dtype=np.uint64).reshape(-1)
    n = off.size
    nb = np.broadcast_to(np.asarray(nbytes, dtype=np.uint64), (n,))
    if (nb % np.uint64(8)).any() or (off % np.uint64(8)).any():
        raise ValueError("ranges must be whole 8-byte words")
    out = np.empty((n, 4), dtype=np.uint64)
    out[:, 0] = off
    out[:, 1] = np.broadcast_to(np.asarray(seed, dtype=np.uint64), (n,))
    out[:, 2] = np.broadcast_to(np.asarray(word0, dtype=np.uint64), (n,))
    out[:, 3] = nb // np.uint64(8)
    if zeros:
        out[:, 3] |= np.uint64(ZEROS)
    return out[out[:, 3] & np.uint64(ZEROS - 1) > 0]


class Page:
    """What one page of a stored object holds: the first `ns` bytes of the
    stream `seed` from word `word0`, then zeros up to the object page; a
    codec page (INT8 form) holds the oracle's encoding of the whole stream
    page instead; a null page is all zeros (ns = 0, codec or not)."""
    __slots__ = ("seed", "word0", "ns", "codec")

    def __init__(self, seed, word0, ns, codec):
        self.seed, self.word0, self.ns, self.codec = seed, word0, ns, codec


class Checker:
    """cfg: the workload; g: its run (pool, objs, slot_of, obj_stride, info,
    objects_on, current_pool_seed); build: DeviceBuild() or HostBuild()."""

    def __init__(self, cfg, g, build):
        self.cfg, self.g, self.build = cfg, g, build
        self.ref = oracle.Layout(cfg.desc)
        ref = self.ref
        assert g.info["num_blocks"] == ref.summary["num_blocks"]
        assert g.info["pool_bytes_used"] == ref.summary["pool_bytes_used"]
        self.Ls = ref.layers
        self.k = ref.k
        self.N = ref.summary["block_size"]
        self.path = ref.summary["path"]
        # every page lies inside one unit: the unified page (path A) or the
        # block stride (path B), so slices of whole units split no page
        self.unit = (ref.summary["unified_page_bytes"] if self.path == 0
                     else ref.summary["block_stride"])
        self.pool_seed = None
        self.overlays = []        # per retrieve wave since the last fill: (rows, masks)
        self.overlay_spans = []   # (lo, hi) byte ranges written since the last fill
        self.stored = {}          # (r, c) -> {(l, j): Page}
        self.obj_fill_seed = None
        self.prefilled = set()
        self.stats = dict(pool_bytes=0, obj_bytes=0, codec_pages=0, waves=0)
        self.pool_exec = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))

    # ------------------------------------------------------------ helpers
    def valid(self, l, j, tokens):
        """Bytes of page j of layer l that a chunk with `tokens` valid tokens
        (None: whole) holds."""
        L = self.Ls[l]
        if not L["is_mla"] or tokens is None:
            return L["page_bytes"]
        rows = min(self.N, max(0, int(tokens) - j * self.N))
        return rows * (L["page_bytes"] // self.N)

    def is_codec(self, l):
        return self.Ls[l]["obj_page_bytes"] != self.Ls[l]["page_bytes"]

    def page_addr(self, l, block):
        L = self.Ls[l]
        return L["pool_offset"] + int(block) * L["stride"]

    def _check_not_overlaid(self, lo, hi):
        for a, b in self.overlay_spans:
            if a < hi and lo < b:
                raise NotImplementedError("a store reads a page retrieved since the last fill; "
                                          "this checker does not model that")

    # ------------------------------------------------------------ waves
    def on_wave(self, i, w):
        g = self.g
        if w.op == "store" and w.pool_seed is not None:
            self.overlays, self.overlay_spans = [], []
        self.pool_seed = g.current_pool_seed
        slots = sorted({g.slot_of[rc] for rc in w.chunks})
        tasks = []
        if w.op == "store":
            for n, rc in enumerate(w.chunks):
                pages = {}
                toks = None if w.chunk_tokens is None else int(w.chunk_tokens[n])
                for l, L in enumerate(self.Ls):
                    for j in range(self.k):
                        bid = int(w.ids[n, L["kv_group"], j])
                        codec = self.is_codec(l)
                        if bid == W.NULL_BLOCK:
                            pages[(l, j)] = Page(0, 0, 0, codec)
                            continue
                        a = self.page_addr(l, bid)
                        v = L["page_bytes"] if codec else self.valid(l, j, toks)
                        self._check_not_overlaid(a, a + v)
                        pages[(l, j)] = Page(self.pool_seed, a // 8, v, codec)
                        if codec:
                            tasks.append(("store", rc, l, j, pages[(l, j)]))
                self.stored[rc] = pages
        else:
            rows, masks = [], []
            for n, rc in enumerate(w.chunks):
                toks = None if w.chunk_tokens is None else int(w.chunk_tokens[n])
                for l, L in enumerate(self.Ls):
                    o = L["obj_group"]
                    for j in range(self.k):
                        bid = int(w.ids[n, L["kv_group"], j])
                        if bid == W.NULL_BLOCK:
                            continue
                        dst = self.page_addr(l, bid)
                        if self.is_codec(l):
                            masks.append((dst, L["page_bytes"]))
                            tasks.append(("retrieve", rc, l, j, dst))
                            self.overlay_spans.append((dst, dst + L["page_bytes"]))
                            continue
                        v = self.valid(l, j, toks)
                        self.overlay_spans.append((dst, dst + v))
                        if rc in self.stored:
                            p = self.stored[rc][(l, j)]
                            ns = min(p.ns, v)
                            rows.append(_rows(dst, p.seed, p.word0, ns))
                            rows.append(_rows(dst + ns, 0, 0, v - ns, zeros=True))
                        else:
                            seed = W.derive_seed(W.object_seed(self.cfg, *rc), o)
                            lo = L["obj_offset"] + j * L["obj_page_bytes"]
                            rows.append(_rows(dst, seed, lo // 8, v))
            table = np.concatenate(rows) if rows else np.zeros((0, 4), np.uint64)
            self.overlays.append((table, masks))
        self.check_pool(i, w)
        self.check_objects(slots, f"wave {i} ({w.op})")
        self.check_codec(tasks, i)
        self.stats["waves"] += 1

    # ------------------------------------------------------------ pool
    def check_pool(self, i, w):
        g = self.g
        pool = g.pool
        total = pool.numel()
        step = max(self.unit, self.build.slice_bytes // self.unit * self.unit)
        E = torch.empty(min(step, total), dtype=torch.uint8, device=pool.device)
        for lo in range(0, total, step):
            hi = min(total, lo + step)
            e = E[: hi - lo]
            self.build.fill(e, self.pool_seed, lo)
            for table, masks in self.overlays:
                if table.shape[0]:
                    dst = table[:, 0]
                    nbytes = (table[:, 3] & np.uint64(ZEROS - 1)) * np.uint64(8)
                    inside = (dst >= np.uint64(lo)) & (dst < np.uint64(hi))
                    if ((dst[inside] + nbytes[inside]) > np.uint64(hi)).any():
                        raise AssertionError("a page straddles a slice boundary")
                    part = table[inside].copy()
                    part[:, 0] -= np.uint64(lo)
                    self.build.fill_rows(e, part)
                for dst, nb in masks:
                    if lo <= dst < hi:
                        assert dst + nb <= hi, "a page straddles a slice boundary"
                        e[dst - lo: dst - lo + nb].copy_(pool[dst: dst + nb])
            self.build.sync()
            if not torch.equal(e, pool[lo:hi]):
                bad = (e != pool[lo:hi]).nonzero()
                first = lo + int(bad[0, 0])
                raise AssertionError(f"wave {i} ({w.op}): pool differs at byte {first} "
                                     f"({bad.shape[0]} bytes in [{lo}, {hi}))")
            self.stats["pool_bytes"] += hi - lo
        del E

    # ------------------------------------------------------------ objects
    def set_object_fill(self, seed):
        self.obj_fill_seed = seed

    def check_objects(self, slots, what):
        """Every byte of the given slots (runs of consecutive slots at a time)."""
        g = self.g
        rc_of = {s: rc for rc, s in g.slot_of.items()}
        for o in range(self.ref.O):
            stride = g.obj_stride[o]
            ob = self.ref.obj_bytes(o)
            buf = g.objs[o]
            per = max(1, self.build.obj_batch_bytes // stride)
            runs, cur = [], []
            for s in slots:
                if cur and (s != cur[-1] + 1 or len(cur) == per):
                    runs.append(cur)
                    cur = []
                cur.append(s)
            if cur:
                runs.append(cur)
            fill_seed = W.derive_seed(self.obj_fill_seed, o)
            for run in runs:
                s0, m = run[0], len(run)
                e = torch.empty(m * stride, dtype=torch.uint8, device=self.build.device)
                self.build.fill(e, fill_seed, s0 * stride)
                base, pages, masks = [], [], []
                for b, s in enumerate(run):
                    rc = rc_of[s]
                    at = b * stride
                    if rc in self.stored:
                        base.append(_rows(at, 0, 0, ob, zeros=True))
                        for l, L in enumerate(self.Ls):
                            if L["obj_group"] != o:
                                continue
                            for j in range(self.k):
                                p = self.stored[rc][(l, j)]
                                lo = at + L["obj_offset"] + j * L["obj_page_bytes"]
                                if p.codec and p.ns:
                                    masks.append((lo, L["obj_page_bytes"]))
                                elif p.ns:
                                    pages.append(_rows(lo, p.seed, p.word0, p.ns))
                    elif rc in self.prefilled:
                        seed = W.derive_seed(W.object_seed(self.cfg, *rc), o)
                        base.append(_rows(at, seed, 0, ob))
                for part in (base, pages):
                    if part:
                        self.build.fill_rows(e, np.concatenate(part))
                got = buf[s0 * stride: (s0 + m) * stride]
                if got.device != e.device:
                    got = got.to(e.device)
                for lo, nb in masks:
                    e[lo: lo + nb].copy_(got[lo: lo + nb])
                self.build.sync()
                if not torch.equal(e, got):
                    bad = (e != got).nonzero()
                    at = int(bad[0, 0])
                    raise AssertionError(f"{what}: object group {o} slot {s0 + at // stride} "
                                         f"differs at byte {at % stride} ({bad.shape[0]} bytes)")
                self.stats["obj_bytes"] += m * stride
                del e, got

    # ------------------------------------------------------------ codec
    def check_codec(self, tasks, i):
        if not tasks:
            return
        g, ref = self.g, self.ref

        def obj_slice(rc, o, lo, n):
            s = g.slot_of[rc]
            t = g.objs[o][s * g.obj_stride[o] + lo: s * g.obj_stride[o] + lo + n]
            return t.cpu().numpy().copy()

        def one(task):
            op, rc, l, j, x = task
            L = self.Ls[l]
            o = L["obj_group"]
            lo = L["obj_offset"] + j * L["obj_page_bytes"]
            if op == "store":
                src = W.fill_bytes(x.seed, x.word0 * 8, L["page_bytes"])
                want = ref.codec_page(src, True, l)
                got = obj_slice(rc, o, lo, L["obj_page_bytes"])
            else:
                if rc in self.stored:
                    p = self.stored[rc][(l, j)]
                    if p.ns == 0:
                        obj = np.zeros(L["obj_page_bytes"], np.uint8)
                    else:
                        obj = ref.codec_page(W.fill_bytes(p.seed, p.word0 * 8,
                                                          L["page_bytes"]), True, l)
                else:
                    seed = W.derive_seed(W.object_seed(self.cfg, *rc), o)
                    obj = W.fill_bytes(seed, lo, L["obj_page_bytes"])
                want = ref.codec_page(obj, False, l)
                got = g.pool[x: x + L["page_bytes"]].cpu().numpy()
            return np.array_equal(got, want), task[:4]

        bad = [t for ok, t in self.pool_exec.map(one, tasks) if not ok]
        assert not bad, f"wave {i}: {len(bad)} codec pages differ from the oracle, e.g. {bad[:3]}"
        self.stats["codec_pages"] += len(tasks)


