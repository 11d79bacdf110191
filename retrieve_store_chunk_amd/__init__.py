"""Python binding of libhkv: chunk store/retrieve for hybrid KDA+MLA caches.

Argument marshalling only: every step runs in the C ABI library
(include/hkv.h) and its HIP kernels.  The functions carry the C names.
Device buffers are passed as integer addresses (e.g. ``tensor.data_ptr()``)
and streams as integer ``hipStream_t`` handles (e.g.
``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is not built, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhkv.so")

HKV_OK = 0
HKV_E_ARG = -1
HKV_E_COVER = -2
HKV_E_CHUNK = -3
HKV_E_BATCH = -4
HKV_E_POOL = -5
HKV_E_RANGE = -6
HKV_E_ALIAS = -7
HKV_E_ALIGN = -8
HKV_E_WORKSPACE = -9
HKV_E_HIP = -10
HKV_E_CAPTURE = -11

STATUS_NAMES = {0: "HKV_OK", -1: "HKV_E_ARG", -2: "HKV_E_COVER", -3: "HKV_E_CHUNK",
                -4: "HKV_E_BATCH", -5: "HKV_E_POOL", -6: "HKV_E_RANGE", -7: "HKV_E_ALIAS",
                -8: "HKV_E_ALIGN", -9: "HKV_E_WORKSPACE", -10: "HKV_E_HIP",
                -11: "HKV_E_CAPTURE"}

i32, i64, u32, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p


class hkv_model(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("is_mla", ctypes.POINTER(ctypes.c_uint8)),
                ("kda_heads", i32), ("kda_head_dim", i32), ("kda_state_bytes", i32),
                ("conv_dim", i32), ("conv_kernel", i32), ("conv_bytes", i32),
                ("mla_width", i32), ("mla_bytes", i32)]


class hkv_layout_desc(ctypes.Structure):
    _fields_ = [("model", hkv_model), ("block_size", i64), ("chunk_min_tokens", i64),
                ("strict_chunk_multiple", i32), ("path", i32),
                ("separate_object_groups", i32), ("kv_group_of_layer", ctypes.POINTER(i32)),
                ("pool_bytes", u64), ("max_num_batched_tokens", i64), ("tile_bytes", u64),
                ("max_workgroups", u32), ("kda_codec", i32)]


class hkv_layout_info(ctypes.Structure):
    _fields_ = [("block_size", i64), ("chunk_tokens", i64), ("blocks_per_chunk", i32),
                ("n_layers", i32), ("n_kv_groups", i32), ("n_obj_groups", i32),
                ("num_blocks", i64), ("path", i32), ("n_slabs", i32),
                ("unified_page_bytes", u64), ("block_stride", u64), ("pool_bytes_used", u64),
                ("obj_bytes", u64 * 2), ("chunk_payload_bytes", u64), ("kda_codec", i32)]


class hkv_layer_info(ctypes.Structure):
    _fields_ = [("is_mla", i32), ("kv_group", i32), ("obj_group", i32), ("slot", i32),
                ("page_bytes", u64), ("reserved_bytes", u64), ("pool_offset", u64),
                ("stride", u64), ("obj_offset", u64), ("obj_page_bytes", u64)]


HKV_NULL_BLOCK = -1


class hkv_chunk_batch(ctypes.Structure):
    _fields_ = [("n_chunks", i32), ("block_ids", ctypes.POINTER(i32)),
                ("objects", ctypes.POINTER(vp)), ("chunk_tokens", ctypes.POINTER(i32)),
                ("engine", i32)]


HKV_ENGINE_KERNEL = 0
HKV_ENGINE_DMA = 1

HKV_OP_STORE = 0
HKV_OP_RETRIEVE = 1


def one_hip_runtime() -> None:
    """A process must hold one HIP runtime.  PyTorch-ROCm ships its own copy,
    which its libraries load by file name; if libhkv.so were loaded first it
    would bring the system runtime and torch would then load a second one
    (each sees the GPU alone, and device memory of one is not usable from the
    other).  Importing torch first makes libhkv bind to torch's runtime."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads a build of libhkv and declares its signatures."""
    one_hip_runtime()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback")
    L = ctypes.CDLL(path)
    L.hkv_unified_block_size.restype = i32
    L.hkv_unified_block_size.argtypes = [ctypes.POINTER(hkv_model), i32, ctypes.POINTER(i64)]
    L.hkv_layout_init.restype = i32
    L.hkv_layout_init.argtypes = [ctypes.POINTER(hkv_layout_desc), ctypes.POINTER(vp)]
    L.hkv_layout_destroy.restype = None
    L.hkv_layout_destroy.argtypes = [vp]
    L.hkv_layout_info_get.restype = i32
    L.hkv_layout_info_get.argtypes = [vp, ctypes.POINTER(hkv_layout_info)]
    L.hkv_layer_info_get.restype = i32
    L.hkv_layer_info_get.argtypes = [vp, i32, ctypes.POINTER(hkv_layer_info)]
    L.hkv_workspace_size.restype = i32
    L.hkv_workspace_size.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.hkv_store_chunks.restype = i32
    L.hkv_store_chunks.argtypes = [vp, vp, ctypes.POINTER(hkv_chunk_batch), vp,
                                   ctypes.c_size_t, vp]
    L.hkv_retrieve_chunks.restype = i32
    L.hkv_retrieve_chunks.argtypes = [vp, vp, ctypes.POINTER(hkv_chunk_batch), vp,
                                      ctypes.c_size_t, vp]
    L.hkv_move_chunks_noalloc.restype = i32
    L.hkv_move_chunks_noalloc.argtypes = [vp, i32, vp, ctypes.POINTER(hkv_chunk_batch), vp]
    L.hkv_layout_fingerprint.restype = i32
    L.hkv_layout_fingerprint.argtypes = [vp, ctypes.POINTER(u64)]
    L.hkv_chunk_keys.restype = i32
    L.hkv_chunk_keys.argtypes = [vp, ctypes.POINTER(i32), i64, i32, u64, u64,
                                 ctypes.POINTER(u64), ctypes.POINTER(u64), i32,
                                 ctypes.POINTER(i64)]
    L.hkv_last_error.restype = ctypes.c_char_p
    L.hkv_last_error.argtypes = []
    return L


lib = _load()


class HkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib.hkv_last_error().decode(errors="replace")
        super().__init__(f"{what} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != HKV_OK:
        raise HkvError(status, what)


def hkv_last_error() -> str:
    return lib.hkv_last_error().decode(errors="replace")


def _model(desc: dict, keep: list) -> hkv_model:
    is_mla = (ctypes.c_uint8 * len(desc["is_mla"]))(*[1 if x else 0 for x in desc["is_mla"]])
    keep.append(is_mla)
    return hkv_model(len(desc["is_mla"]), ctypes.cast(is_mla, ctypes.POINTER(ctypes.c_uint8)),
                     desc["kda_heads"], desc["kda_head_dim"], desc["kda_state_bytes"],
                     desc["conv_dim"], desc["conv_kernel"], desc["conv_bytes"],
                     desc["mla_width"], desc["mla_bytes"])


def hkv_unified_block_size(desc: dict, align_tokens: int = 16) -> int:
    """N for the model part of a layout description dict."""
    keep = []
    m = _model(desc, keep)
    out = i64()
    _check(lib.hkv_unified_block_size(ctypes.byref(m), align_tokens, ctypes.byref(out)),
           "hkv_unified_block_size")
    return out.value


def hkv_layout_init(desc: dict) -> int:
    """Builds a layout from a description dict; returns the opaque handle."""
    keep = []
    d = hkv_layout_desc()
    d.model = _model(desc, keep)
    d.block_size = desc.get("block_size", 0)
    d.chunk_min_tokens = desc.get("chunk_min_tokens", 1)
    d.strict_chunk_multiple = int(desc.get("strict_chunk_multiple", 0))
    d.path = desc["path"]
    d.separate_object_groups = int(desc.get("separate_object_groups", 1))
    kvg = desc.get("kv_group_of_layer")
    if kvg is not None:
        arr = (i32 * len(kvg))(*kvg)
        keep.append(arr)
        d.kv_group_of_layer = ctypes.cast(arr, ctypes.POINTER(i32))
    d.pool_bytes = desc["pool_bytes"]
    d.max_num_batched_tokens = desc.get("max_num_batched_tokens", 0)
    d.tile_bytes = desc.get("tile_bytes", 0)
    d.max_workgroups = desc.get("max_workgroups", 0)
    d.kda_codec = int(desc.get("kda_codec", 0))
    h = vp()
    _check(lib.hkv_layout_init(ctypes.byref(d), ctypes.byref(h)), "hkv_layout_init")
    return h.value


def hkv_layout_destroy(handle: int) -> None:
    lib.hkv_layout_destroy(handle)


def hkv_layout_info_get(handle: int) -> dict:
    out = hkv_layout_info()
    _check(lib.hkv_layout_info_get(handle, ctypes.byref(out)), "hkv_layout_info_get")
    d = {name: getattr(out, name) for name, _ in hkv_layout_info._fields_}
    d["obj_bytes"] = [int(out.obj_bytes[0]), int(out.obj_bytes[1])]
    return d


def hkv_layer_info_get(handle: int, layer: int) -> dict:
    out = hkv_layer_info()
    _check(lib.hkv_layer_info_get(handle, layer, ctypes.byref(out)), "hkv_layer_info_get")
    return {name: getattr(out, name) for name, _ in hkv_layer_info._fields_}


def hkv_workspace_size(handle: int, max_chunks: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.hkv_workspace_size(handle, max_chunks, ctypes.byref(out)), "hkv_workspace_size")
    return out.value


def hkv_layout_fingerprint(handle: int) -> int:
    out = u64()
    _check(lib.hkv_layout_fingerprint(handle, ctypes.byref(out)), "hkv_layout_fingerprint")
    return out.value


def hkv_chunk_keys(handle: int, tokens, hash_block_tokens: int = 0, root: int = 0,
                   rank_tag: int = 0, info: dict | None = None):
    """Returns (prefix_hashes [n_tokens // h] uint64, keys [n_chunks][O] uint64).
    `info` (the layout's hkv_layout_info_get) may be passed to skip the query."""
    import numpy as np
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    info = info or hkv_layout_info_get(handle)
    h = hash_block_tokens or info["block_size"]
    n_fine = toks.size // h if h > 0 else 0
    n_chunks = toks.size // info["chunk_tokens"]
    prefix = np.zeros(max(1, n_fine), dtype=np.uint64)
    keys = np.zeros((max(1, n_chunks), info["n_obj_groups"]), dtype=np.uint64)
    got = i64()
    p_u64 = ctypes.POINTER(u64)
    _check(lib.hkv_chunk_keys(handle, toks.ctypes.data_as(ctypes.POINTER(i32)), toks.size,
                              hash_block_tokens, root & (2**64 - 1), rank_tag & (2**64 - 1),
                              prefix.ctypes.data_as(p_u64), keys.ctypes.data_as(p_u64),
                              n_chunks, ctypes.byref(got)), "hkv_chunk_keys")
    return prefix[:n_fine], keys[:got.value]


def _batch(handle, block_ids, objects, info=None, chunk_tokens=None, engine=HKV_ENGINE_KERNEL):
    """block_ids: int32 array [n][G][k]; objects: flat sequence of n*O device
    addresses (chunk-major); chunk_tokens: None or int32 [n]; engine:
    HKV_ENGINE_KERNEL or HKV_ENGINE_DMA.  Shapes are checked against the
    layout so the library never reads past the host arrays."""
    import numpy as np
    ids = np.ascontiguousarray(block_ids, dtype=np.int32)
    n = int(ids.shape[0]) if ids.ndim else 0
    toks = None
    if chunk_tokens is not None:
        toks = np.ascontiguousarray(chunk_tokens, dtype=np.int32)
        if toks.shape != (n,):
            raise ValueError(f"chunk_tokens must have shape ({n},), got {toks.shape}")
    if handle:
        info = info or hkv_layout_info_get(handle)
        want = (n, info["n_kv_groups"], info["blocks_per_chunk"])
        if ids.shape != want:
            raise ValueError(f"block_ids must have shape {want}, got {ids.shape}")
        if len(objects) != n * info["n_obj_groups"]:
            raise ValueError(f"need {n * info['n_obj_groups']} object addresses, "
                             f"got {len(objects)}")
    addrs = (vp * max(1, len(objects)))(*[int(a) for a in objects])
    b = hkv_chunk_batch(n, ids.ctypes.data_as(ctypes.POINTER(i32)),
                        ctypes.cast(addrs, ctypes.POINTER(vp)),
                        None if toks is None else toks.ctypes.data_as(ctypes.POINTER(i32)),
                        int(engine))
    return b, (ids, addrs, toks)


def hkv_store_chunks(handle: int, pool_ptr: int, block_ids, objects, workspace_ptr: int,
                     ws_bytes: int, stream: int = 0, info: dict | None = None,
                     chunk_tokens=None, engine: int = HKV_ENGINE_KERNEL) -> None:
    b, keep = _batch(handle, block_ids, objects, info, chunk_tokens, engine)
    _check(lib.hkv_store_chunks(handle, pool_ptr, ctypes.byref(b), workspace_ptr, ws_bytes,
                                stream), "hkv_store_chunks")
    del keep


def hkv_retrieve_chunks(handle: int, pool_ptr: int, block_ids, objects, workspace_ptr: int,
                        ws_bytes: int, stream: int = 0, info: dict | None = None,
                        chunk_tokens=None, engine: int = HKV_ENGINE_KERNEL) -> None:
    b, keep = _batch(handle, block_ids, objects, info, chunk_tokens, engine)
    _check(lib.hkv_retrieve_chunks(handle, pool_ptr, ctypes.byref(b), workspace_ptr, ws_bytes,
                                   stream), "hkv_retrieve_chunks")
    del keep


def hkv_move_chunks_noalloc(handle: int, op: int, pool_ptr: int, block_ids, objects,
                            stream: int = 0, info: dict | None = None,
                            chunk_tokens=None) -> None:
    """op: HKV_OP_STORE or HKV_OP_RETRIEVE.  No workspace: the library keeps
    the layout's tables in its static device scratch."""
    b, keep = _batch(handle, block_ids, objects, info, chunk_tokens, HKV_ENGINE_KERNEL)
    _check(lib.hkv_move_chunks_noalloc(handle, op, pool_ptr, ctypes.byref(b), stream),
           "hkv_move_chunks_noalloc")
    del keep


def status_of(fn, *args) -> int:
    """Calls one of the wrappers above and returns its status instead of
    raising (for tests of error paths)."""
    try:
        fn(*args)
        return HKV_OK
    except HkvError as e:
        return e.status


class Layout:
    """Owns a layout handle; exposes its summary and per-layer placements."""

    def __init__(self, desc: dict):
        self._lib = lib  # the build that owns the handle
        self.handle = hkv_layout_init(desc)
        self.info = hkv_layout_info_get(self.handle)
        self.layers = [hkv_layer_info_get(self.handle, l) for l in range(self.info["n_layers"])]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and getattr(self, "_lib", None) is not None:
            self._lib.hkv_layout_destroy(h)
            self.handle = None

    @property
    def G(self) -> int:
        return self.info["n_kv_groups"]

    @property
    def O(self) -> int:
        return self.info["n_obj_groups"]

    @property
    def k(self) -> int:
        return self.info["blocks_per_chunk"]

    def workspace_size(self, max_chunks: int) -> int:
        return hkv_workspace_size(self.handle, max_chunks)

    def fingerprint(self) -> int:
        return hkv_layout_fingerprint(self.handle)

    def chunk_keys(self, tokens, hash_block_tokens=0, root=0, rank_tag=0):
        return hkv_chunk_keys(self.handle, tokens, hash_block_tokens, root, rank_tag,
                              info=self.info)

    def store(self, pool_ptr, block_ids, objects, ws_ptr, ws_bytes, stream=0,
              chunk_tokens=None, engine=HKV_ENGINE_KERNEL):
        hkv_store_chunks(self.handle, pool_ptr, block_ids, objects, ws_ptr, ws_bytes, stream,
                         info=self.info, chunk_tokens=chunk_tokens, engine=engine)

    def retrieve(self, pool_ptr, block_ids, objects, ws_ptr, ws_bytes, stream=0,
                 chunk_tokens=None, engine=HKV_ENGINE_KERNEL):
        hkv_retrieve_chunks(self.handle, pool_ptr, block_ids, objects, ws_ptr, ws_bytes, stream,
                            info=self.info, chunk_tokens=chunk_tokens, engine=engine)

    def move_noalloc(self, op, pool_ptr, block_ids, objects, stream=0, chunk_tokens=None):
        hkv_move_chunks_noalloc(self.handle, op, pool_ptr, block_ids, objects, stream,
                                info=self.info, chunk_tokens=chunk_tokens)
