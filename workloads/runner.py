"""Runs a workload through the HIP library: torch for device memory and
streams, the product binding for every store/retrieve.  No oracle here.

Object storage: one device tensor per object group with one slot per
(request, chunk) that any phase touches; slot rows are 256-byte aligned.
"""
from __future__ import annotations

import numpy as np
import torch

import retrieve_store_chunk_amd as hkv
import workloads as W


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


class GpuWorkload:
    def __init__(self, cfg: W.Config, device: str = "cuda:0", tile_bytes: int = 0,
                 max_workgroups: int = 0, stream: torch.cuda.Stream | None = None,
                 objects: str = "device", retrieve_engine: str | None = None,
                 entry: str = "workspace"):
        """objects: "device" (HBM) or "host" (pinned host memory, which the
        GPU reads and writes over the host link).  retrieve_engine: "kernel"
        or "dma" (default: the workload's own choice, else "kernel").
        entry: "workspace" (hkv_store_chunks / hkv_retrieve_chunks) or
        "noalloc" (hkv_move_chunks_noalloc; kernel engine only)."""
        if objects not in ("device", "host"):
            raise ValueError("objects must be 'device' or 'host'")
        if entry not in ("workspace", "noalloc"):
            raise ValueError("entry must be 'workspace' or 'noalloc'")
        self.entry = entry
        self.cfg = cfg
        self.objects_on = objects
        engine = retrieve_engine or cfg.extra.get("retrieve_engine", "kernel")
        if engine not in ("kernel", "dma"):
            raise ValueError("retrieve_engine must be 'kernel' or 'dma'")
        if entry == "noalloc" and engine == "dma":
            raise ValueError("the no-allocation entry point runs the kernels only")
        self.retrieve_engine = hkv.HKV_ENGINE_DMA if engine == "dma" else hkv.HKV_ENGINE_KERNEL
        self.device = torch.device(device)
        desc = dict(cfg.desc, tile_bytes=tile_bytes, max_workgroups=max_workgroups)
        self.layout = hkv.Layout(desc)
        info = self.layout.info
        self.info = info
        kda_groups = {L["kv_group"] for L in self.layout.layers if not L["is_mla"]}
        self.waves = W.plan_waves(cfg, info["num_blocks"], self.layout.G, self.layout.k,
                                  kda_groups, info["block_size"], info["chunk_tokens"])
        self.stream = stream if stream is not None else torch.cuda.Stream(device=self.device)
        # object slots
        self.slot_of = {}
        for ph in cfg.phases:
            for rc in ph.chunks:
                self.slot_of.setdefault(rc, len(self.slot_of))
        n_slots = len(self.slot_of)
        self.obj_stride = [_align(max(1, info["obj_bytes"][o])) for o in range(self.layout.O)]
        self.pool = torch.empty(_align(info["pool_bytes_used"]), dtype=torch.uint8,
                                device=self.device)
        if objects == "device":
            self.objs = [torch.empty(n_slots * self.obj_stride[o], dtype=torch.uint8,
                                     device=self.device) for o in range(self.layout.O)]
        else:
            self.objs = [torch.empty(n_slots * self.obj_stride[o], dtype=torch.uint8,
                                     pin_memory=True) for o in range(self.layout.O)]
        max_chunks = max((len(w.chunks) for w in self.waves), default=0)
        self.ws_bytes = self.layout.workspace_size(max_chunks)
        self.ws = torch.empty(max(256, self.ws_bytes), dtype=torch.uint8, device=self.device)
        # duplex workloads run their retrieves on a second stream, with a
        # workspace of their own, beside the stores
        self.duplex = bool(cfg.extra.get("duplex"))
        self.stream2 = torch.cuda.Stream(device=self.device) if self.duplex else self.stream
        self.ws2 = (torch.empty(max(256, self.ws_bytes), dtype=torch.uint8, device=self.device)
                    if self.duplex else self.ws)
        self.pool_seed_of = {}   # (r, c) -> seed of the pool its store read
        self.store_ids = {}      # (r, c) -> [G][k] block ids its store read

    # ------------------------------------------------------------ addresses
    def object_ptrs(self, chunks) -> list:
        out = []
        for rc in chunks:
            s = self.slot_of[rc]
            for o in range(self.layout.O):
                out.append(self.objs[o].data_ptr() + s * self.obj_stride[o])
        return out

    def object_view(self, rc, o) -> torch.Tensor:
        s = self.slot_of[rc]
        return self.objs[o][s * self.obj_stride[o]: s * self.obj_stride[o]
                            + self.info["obj_bytes"][o]]

    # ------------------------------------------------------------ fills
    def fill_pool(self, seed: int) -> None:
        with torch.cuda.stream(self.stream):
            W.gpu_fill(self.pool.data_ptr(), self.pool.numel(), seed, 0,
                       self.stream.cuda_stream)

    def fill_objects(self, seed: int) -> None:
        """Every object byte: group o's buffer is the stream derive_seed(seed, o)
        (filled by the GPU in device memory, by the host in pinned memory)."""
        for o in range(self.layout.O):
            if self.objects_on == "device":
                W.gpu_fill(self.objs[o].data_ptr(), self.objs[o].numel(),
                           W.derive_seed(seed, o), 0, self.stream.cuda_stream)
            else:
                self.stream.synchronize()
                self.objs[o].numpy()[:] = W.fill_bytes(W.derive_seed(seed, o), 0,
                                                       self.objs[o].numel())

    def prefill_objects(self) -> None:
        """Objects that a retrieve reads without an earlier store in this run
        hold seeded bytes: object group o of (r, c) is the stream
        derive_seed(object_seed(r, c), o)."""
        for w in self.waves:
            if w.op == "retrieve" and w.prefilled_objects:
                for rc in w.chunks:
                    for o in range(self.layout.O):
                        v = self.object_view(rc, o)
                        seed = W.derive_seed(W.object_seed(self.cfg, *rc), o)
                        if self.objects_on == "device":
                            W.gpu_fill(v.data_ptr(), v.numel(), seed, 0, self.stream.cuda_stream)
                        else:
                            self.stream.synchronize()
                            v.numpy()[:] = W.fill_bytes(seed, 0, v.numel())

    # ------------------------------------------------------------ calls
    def stream_of(self, w: W.Wave) -> torch.cuda.Stream:
        """The stream a wave runs on: the second one for a duplex retrieve."""
        return self.stream2 if (self.duplex and w.op == "retrieve") else self.stream

    def run_wave(self, w: W.Wave) -> None:
        ptrs = self.object_ptrs(w.chunks)
        if self.entry == "noalloc":
            op = hkv.HKV_OP_STORE if w.op == "store" else hkv.HKV_OP_RETRIEVE
            self.layout.move_noalloc(op, self.pool.data_ptr(), w.ids, ptrs,
                                     self.stream_of(w).cuda_stream, chunk_tokens=w.chunk_tokens)
            return
        fn = self.layout.store if w.op == "store" else self.layout.retrieve
        second = self.duplex and w.op == "retrieve"
        ws = self.ws2 if second else self.ws
        engine = self.retrieve_engine if w.op == "retrieve" else hkv.HKV_ENGINE_KERNEL
        fn(self.pool.data_ptr(), w.ids, ptrs, ws.data_ptr(), self.ws_bytes,
           self.stream_of(w).cuda_stream, chunk_tokens=w.chunk_tokens, engine=engine)

    def run_all(self, on_wave=None) -> None:
        """Every wave in order.  A store wave with a pool seed first refills
        the pool with it.  Records, per stored chunk, the seed of the pool
        it read and its block ids."""
        self.prefill_objects()
        if self.duplex:
            self._run_all_duplex(on_wave)
            return
        for i, w in enumerate(self.waves):
            if w.op == "store" and w.pool_seed is not None:
                self.fill_pool(w.pool_seed)
                self.current_pool_seed = w.pool_seed
            if w.op == "store":
                for n, rc in enumerate(w.chunks):
                    self.pool_seed_of[rc] = self.current_pool_seed
                    self.store_ids[rc] = w.ids[n].copy()
            self.run_wave(w)
            if on_wave is not None:
                self.stream.synchronize()
                on_wave(i, w)

    def _run_all_duplex(self, on_wave) -> None:
        """Duplex: one pool fill, then every wave at once (stores on the
        first stream, retrieves on the second, which waits for the fills);
        on_wave sees each wave after all have finished."""
        seeds = [w.pool_seed for w in self.waves if w.op == "store" and w.pool_seed is not None]
        if len(seeds) > 1:
            raise ValueError("a duplex workload refills its pool once")
        if seeds:
            self.fill_pool(seeds[0])
            self.current_pool_seed = seeds[0]
        self.stream2.wait_stream(self.stream)
        for w in self.waves:
            if w.op == "store":
                for n, rc in enumerate(w.chunks):
                    self.pool_seed_of[rc] = self.current_pool_seed
                    self.store_ids[rc] = w.ids[n].copy()
            self.run_wave(w)
        self.synchronize()
        if on_wave is not None:
            for i, w in enumerate(self.waves):
                on_wave(i, w)

    def synchronize(self) -> None:
        self.stream.synchronize()
        if self.duplex:
            self.stream2.synchronize()

    current_pool_seed = None

    def init_pool(self) -> int:
        seed = W.initial_pool_seed(self.cfg)
        self.fill_pool(seed)
        self.current_pool_seed = seed
        return seed

    def payload_bytes(self, waves=None) -> int:
        waves = self.waves if waves is None else waves
        return sum(len(w.chunks) for w in waves) * self.info["chunk_payload_bytes"]

    def host_pool(self) -> np.ndarray:
        self.stream.synchronize()
        return self.pool[: self.info["pool_bytes_used"]].cpu().numpy()

    def host_object(self, rc, o) -> np.ndarray:
        self.stream.synchronize()
        return self.object_view(rc, o).cpu().numpy().copy()
