"""CPU: the every-byte checker of the full-size GPU test (tests/fullsize_check.py),
run against the oracle on small workloads.

A stand-in for the GPU run executes the same waves with the oracle on host
tensors; the checker then rebuilds its expected bytes on the host.  It must
pass on a correct run, and fail on each planted corruption of the run's
buffers: a byte written in padding, group slack or an untargeted block, in
the bytes between object slots, past a partial chunk's rows, in a store's
source page, or in an INT8 code.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.fullsize_check import Checker, HostBuild


def _align(x, a=256):
    return (x + a - 1) // a * a


class OracleRun:
    """What the checker reads of workloads.runner.GpuWorkload, with every
    wave run by the oracle on host tensors."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.ref = oracle.Layout(cfg.desc)
        s = self.ref.summary
        self.info = {"num_blocks": s["num_blocks"], "pool_bytes_used": s["pool_bytes_used"],
                     "obj_bytes": [s["obj_bytes0"], s["obj_bytes1"]]}
        kda_groups = {L["kv_group"] for L in self.ref.layers if not L["is_mla"]}
        self.waves = W.plan_waves(cfg, s["num_blocks"], self.ref.G, self.ref.k, kda_groups,
                                  s["block_size"], s["chunk_tokens"])
        self.slot_of = {}
        for ph in cfg.phases:
            for rc in ph.chunks:
                self.slot_of.setdefault(rc, len(self.slot_of))
        self.obj_stride = [_align(max(1, self.ref.obj_bytes(o))) for o in range(self.ref.O)]
        self.pool = torch.empty(_align(s["pool_bytes_used"]), dtype=torch.uint8)
        self.objs = [torch.empty(len(self.slot_of) * self.obj_stride[o], dtype=torch.uint8)
                     for o in range(self.ref.O)]
        self.objects_on = "device"
        self.current_pool_seed = None
        self.duplex = bool(cfg.extra.get("duplex"))

    def fill_pool(self, seed):
        self.pool.numpy()[:] = W.fill_bytes(seed, 0, self.pool.numel())
        self.current_pool_seed = seed

    def init_pool(self):
        self.fill_pool(W.initial_pool_seed(self.cfg))

    def fill_objects(self, seed):
        for o, t in enumerate(self.objs):
            t.numpy()[:] = W.fill_bytes(W.derive_seed(seed, o), 0, t.numel())

    def view(self, rc, o):
        s = self.slot_of[rc]
        return self.objs[o].numpy()[s * self.obj_stride[o]:
                                    s * self.obj_stride[o] + self.ref.obj_bytes(o)]

    def synchronize(self):
        pass

    def _run(self, w):
        objs = [[self.view(rc, o) for o in range(self.ref.O)] for rc in w.chunks]
        fn = self.ref.store if w.op == "store" else self.ref.retrieve
        fn(self.pool.numpy(), w.ids, objs, chunk_tokens=w.chunk_tokens)

    def run_all(self, on_wave, corrupt=None):
        for w in self.waves:
            if w.op == "retrieve" and w.prefilled_objects:
                for rc in w.chunks:
                    for o in range(self.ref.O):
                        v = self.view(rc, o)
                        v[:] = W.fill_bytes(W.derive_seed(W.object_seed(self.cfg, *rc), o), 0,
                                            v.size)
        if self.duplex:
            for w in self.waves:
                self._run(w)
            for i, w in enumerate(self.waves):
                if corrupt:
                    corrupt(i, w, self)
                on_wave(i, w)
            return
        for i, w in enumerate(self.waves):
            if w.op == "store" and w.pool_seed is not None:
                self.fill_pool(w.pool_seed)
            self._run(w)
            if corrupt:
                corrupt(i, w, self)
            on_wave(i, w)


def check_run(cfg, corrupt=None):
    run = OracleRun(cfg)
    chk = Checker(cfg, run, HostBuild())
    run.init_pool()
    seed = W.derive_seed(cfg.seed, 77)
    run.fill_objects(seed)
    chk.set_object_fill(seed)
    chk.prefilled = {rc for w in run.waves if w.op == "retrieve" and w.prefilled_objects
                     for rc in w.chunks}
    try:
        run.run_all(chk.on_wave, corrupt)
        chk.check_objects(sorted(run.slot_of.values()), "end of run")
    finally:
        chk.pool_exec.shutdown()
    assert chk.stats["pool_bytes"] == chk.stats["waves"] * run.pool.numel()
    return chk


# ---------------------------------------------------------------- workloads
def tiny():
    return W.make_config("tiny")


def tiny_path_b():
    cfg = copy.deepcopy(tiny())
    cfg.desc["path"] = 1
    cfg.name = "tiny_path_b"
    return cfg


def tiny_codec():
    cfg = copy.deepcopy(tiny())
    cfg.desc["kda_codec"] = 1
    cfg.name = "tiny_codec"
    return cfg


def holes_tails():
    """k = 2 blocks per chunk, KDA snapshots every 2nd block, partial chunks."""
    desc = W._desc([0, 0, 0, 1, 0, 1], 2, 16, 96, 2, 0, 48 * 16 * 576 * 2, chunk_min=32,
                   max_batched=64)
    req = [3, 2, 3, 1]
    tails = {(0, 2): 20, (1, 1): 16, (3, 0): 7}
    chunks = [(r, c) for r, n in enumerate(req) for c in range(n)]
    return W.Config("holes_tails", "holes and tails", desc, req,
                    [W.Phase("store", chunks, snapshot_every=2, tail_tokens=tails),
                     W.Phase("retrieve", chunks, snapshot_every=2, tail_tokens=tails)],
                    seed=0x48B0100)


def prefix_then_tails():
    """A prefilled prefix retrieve, then stores, from one permutation (no refill)."""
    cfg = copy.deepcopy(tiny())
    cfg.name = "prefix_then_tails"
    cfg.requests = [5] + [1] * 6
    cfg.phases = [W.Phase("retrieve", [(0, c) for c in range(5)], prefilled_objects=True),
                  W.Phase("store", [(r, 0) for r in range(1, 7)])]
    cfg.shared_permutation = True
    return cfg


def duplex():
    cfg = prefix_then_tails()
    cfg.name = "duplex"
    cfg.extra = {"duplex": True}
    return cfg


CASES = [tiny, tiny_path_b, tiny_codec, holes_tails, prefix_then_tails, duplex]


@pytest.mark.parametrize("make", CASES, ids=lambda f: f.__name__)
def test_checker_passes_a_correct_run(make):
    chk = check_run(make())
    assert chk.stats["waves"] >= 2
    if make is tiny_codec:
        assert chk.stats["codec_pages"] > 0


# ---------------------------------------------------------------- corruptions
def _first(w, op):
    return w.op == op


def flip(t, at):
    a = t.numpy()
    a[at] ^= 0x5A


def corrupt_padding(i, w, run):
    """Path A: a byte of a retrieved KDA page's padding."""
    if _first(w, "retrieve"):
        L = next(L for L in run.ref.layers if not L["is_mla"])
        b = int(w.ids[0, L["kv_group"], 0])
        flip(run.pool, L["pool_offset"] + b * L["stride"] + L["page_bytes"] + 3)


def corrupt_slack(i, w, run):
    """Path B: a byte of a targeted block's group slack."""
    if _first(w, "retrieve"):
        L = next(L for L in run.ref.layers if not L["is_mla"])
        b = int(w.ids[0, L["kv_group"], 0])
        flip(run.pool, b * run.ref.summary["block_stride"] + L["page_bytes"] + 5)


def corrupt_untargeted(i, w, run):
    """A byte of a block that the wave does not name (the first wave that
    leaves one free)."""
    if getattr(run, "corrupted", False):
        return
    used = set(w.ids.reshape(-1).tolist())
    free = [b for b in range(run.ref.summary["num_blocks"]) if b not in used]
    if free:
        L = run.ref.layers[-1]
        flip(run.pool, L["pool_offset"] + free[0] * L["stride"] + 11)
        run.corrupted = True


def corrupt_between_slots(i, w, run):
    if _first(w, "store"):
        o = 0
        s = run.slot_of[w.chunks[0]]
        flip(run.objs[o], s * run.obj_stride[o] + run.ref.obj_bytes(o))  # first byte past it


def corrupt_object_page(i, w, run):
    if _first(w, "store"):
        flip(run.objs[1], run.slot_of[w.chunks[-1]] * run.obj_stride[1] + 100)


def corrupt_store_source(i, w, run):
    """A store must leave its source pages unchanged."""
    if _first(w, "store"):
        L = run.ref.layers[0]
        b = int(w.ids[0, L["kv_group"], 0])
        if b >= 0:
            flip(run.pool, L["pool_offset"] + b * L["stride"])


def corrupt_past_tail(i, w, run):
    """A retrieve must not write an MLA page's rows past the chunk's tokens."""
    if _first(w, "retrieve") and w.chunk_tokens is not None:
        N = run.ref.summary["block_size"]
        for n, t in enumerate(w.chunk_tokens):
            for l, L in enumerate(run.ref.layers):
                if not L["is_mla"]:
                    continue
                for j in range(run.ref.k):
                    b = int(w.ids[n, L["kv_group"], j])
                    rows = min(N, max(0, int(t) - j * N))
                    if b >= 0 and 0 < rows < N:
                        flip(run.pool, L["pool_offset"] + b * L["stride"] +
                             rows * (L["page_bytes"] // N))
                        return
        raise RuntimeError("no partial page to corrupt")


def corrupt_codec_code(i, w, run):
    if _first(w, "store"):
        L = next(L for L in run.ref.layers if not L["is_mla"])
        s = run.slot_of[w.chunks[0]]
        o = L["obj_group"]
        flip(run.objs[o], s * run.obj_stride[o] + L["obj_offset"] + L["obj_page_bytes"] - 200)


def corrupt_decoded_state(i, w, run):
    if _first(w, "retrieve"):
        L = next(L for L in run.ref.layers if not L["is_mla"])
        b = int(w.ids[0, L["kv_group"], 0])
        flip(run.pool, L["pool_offset"] + b * L["stride"] + L["page_bytes"] - 8)


MUTANTS = [(tiny, corrupt_padding), (tiny_path_b, corrupt_slack),
           (holes_tails, corrupt_untargeted), (prefix_then_tails, corrupt_untargeted), (tiny, corrupt_between_slots),
           (tiny, corrupt_object_page), (tiny, corrupt_store_source),
           (holes_tails, corrupt_past_tail), (tiny_codec, corrupt_codec_code),
           (tiny_codec, corrupt_decoded_state), (duplex, corrupt_object_page)]


@pytest.mark.parametrize("make,corrupt", MUTANTS,
                         ids=lambda x: x.__name__)
def test_checker_catches_a_planted_corruption(make, corrupt):
    with pytest.raises(AssertionError, match="differ"):
        check_run(make(), corrupt)
