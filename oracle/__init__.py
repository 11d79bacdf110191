"""ctypes wrapper of the CPU oracle (libhkvref.so).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product package never imports
this module.  The oracle itself is plain C (hkvref.c); this file only
marshals arguments.

A layout is described by the same plain dict of workload parameters that the
product binding takes (keys listed in ``DESC_KEYS``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB_PATH = os.path.join(HERE, "libhkvref.so")
# HKVREF_LIB names another build of hkvref.c (the tests' sanitized build).
LIB_PATH = os.environ.get("HKVREF_LIB") or DEFAULT_LIB_PATH

DESC_KEYS = (
    "is_mla", "kda_heads", "kda_head_dim", "kda_state_bytes", "conv_dim", "conv_kernel",
    "conv_bytes", "mla_width", "mla_bytes", "block_size", "chunk_min_tokens",
    "strict_chunk_multiple", "path", "separate_object_groups", "kv_group_of_layer",
    "pool_bytes", "max_num_batched_tokens", "kda_codec",
)

OK, E_ARG, E_COVER, E_CHUNK, E_BATCH, E_POOL, E_RANGE, E_ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
NULL_BLOCK = -1

_lib = None


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) and LIB_PATH == DEFAULT_LIB_PATH:
            from . import build as _build  # noqa: F401  (build on first use)
            _build.build()
        _lib = bind(ctypes.CDLL(LIB_PATH))
    return _lib


def bind(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declares the C signatures on a loaded build of hkvref.c."""
    i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    vp = ctypes.c_void_p
    L.hkvref_kda_page_bytes.restype = i64
    L.hkvref_kda_page_bytes.argtypes = [i32] * 6
    L.hkvref_unified_block_size.restype = ctypes.c_int
    L.hkvref_unified_block_size.argtypes = [i64, i64, i64, ctypes.POINTER(i64)]
    L.hkvref_chunk_tokens.restype = ctypes.c_int
    L.hkvref_chunk_tokens.argtypes = [i64, i64, i32, ctypes.POINTER(i64)]
    L.hkvref_layout_init.restype = ctypes.c_int
    L.hkvref_layout_init.argtypes = [i32, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                     i64, i64, i32, i32, i32, vp, u64, i64, i32,
                                     ctypes.POINTER(vp)]
    L.hkvref_layout_free.restype = None
    L.hkvref_layout_free.argtypes = [vp]
    L.hkvref_layout_summary.restype = ctypes.c_int
    L.hkvref_layout_summary.argtypes = [vp, ctypes.POINTER(i64)]
    L.hkvref_layer.restype = ctypes.c_int
    L.hkvref_layer.argtypes = [vp, i32, ctypes.POINTER(i64)]
    L.hkvref_store_chunks.restype = ctypes.c_int
    L.hkvref_store_chunks.argtypes = [vp, vp, i32, vp, vp, vp]
    L.hkvref_retrieve_chunks.restype = ctypes.c_int
    L.hkvref_retrieve_chunks.argtypes = [vp, vp, i32, vp, vp, vp]
    L.hkvref_fingerprint.restype = u64
    L.hkvref_fingerprint.argtypes = [vp]
    L.hkvref_codec_page.restype = ctypes.c_int
    L.hkvref_codec_page.argtypes = [vp, i32, vp, vp]
    L.hkvref_chunk_keys.restype = ctypes.c_int
    L.hkvref_chunk_keys.argtypes = [vp, vp, i64, i32, u64, u64, vp, vp, i32,
                                    ctypes.POINTER(i64)]
    return L


def kda_page_bytes(heads, head_dim, state_bytes, conv_dim, conv_kernel, conv_bytes) -> int:
    return int(lib().hkvref_kda_page_bytes(heads, head_dim, state_bytes, conv_dim,
                                           conv_kernel, conv_bytes))


def unified_block_size(kda_page: int, tok_bytes: int, align: int = 16) -> int:
    out = ctypes.c_int64()
    rc = lib().hkvref_unified_block_size(kda_page, tok_bytes, align, ctypes.byref(out))
    if rc != OK:
        raise OracleError(rc, "unified_block_size")
    return out.value


def chunk_tokens(n: int, chunk_min: int, strict: bool = False) -> int:
    out = ctypes.c_int64()
    rc = lib().hkvref_chunk_tokens(n, chunk_min, int(strict), ctypes.byref(out))
    if rc != OK:
        raise OracleError(rc, "chunk_tokens")
    return out.value


SUMMARY_FIELDS = ("block_size", "chunk_tokens", "blocks_per_chunk", "num_blocks", "n_layers",
                  "n_kv_groups", "n_obj_groups", "path", "n_slabs", "unified_page_bytes",
                  "block_stride", "obj_bytes0", "obj_bytes1", "pool_bytes_used", "kda_codec")
LAYER_FIELDS = ("is_mla", "kv_group", "obj_group", "slot", "page_bytes", "reserved_bytes",
                "pool_offset", "stride", "obj_offset", "obj_page_bytes")


def _ptr_array(objects, n_chunks: int, n_obj: int):
    """objects: [n_chunks][n_obj] numpy uint8 arrays -> (ctypes array, keepalive)."""
    if len(objects) != n_chunks:
        raise ValueError("objects must have one entry per chunk")
    addrs = (ctypes.c_void_p * max(1, n_chunks * n_obj))()
    for c in range(n_chunks):
        if len(objects[c]) != n_obj:
            raise ValueError("each chunk needs one object per object group")
        for o in range(n_obj):
            a = objects[c][o]
            if not (isinstance(a, np.ndarray) and a.dtype == np.uint8 and a.flags.c_contiguous):
                raise TypeError("objects must be C-contiguous uint8 numpy arrays")
            addrs[c * n_obj + o] = a.ctypes.data
    return addrs


class Layout:
    """An oracle layout (owns the C handle)."""

    def __init__(self, desc: dict):
        L = lib()
        self._L = L
        is_mla = np.ascontiguousarray(np.asarray(desc["is_mla"], dtype=np.uint8))
        kvg = desc.get("kv_group_of_layer")
        kvg_arr = None if kvg is None else np.ascontiguousarray(np.asarray(kvg, dtype=np.int32))
        h = ctypes.c_void_p()
        rc = L.hkvref_layout_init(
            len(is_mla), is_mla.ctypes.data,
            desc["kda_heads"], desc["kda_head_dim"], desc["kda_state_bytes"],
            desc["conv_dim"], desc["conv_kernel"], desc["conv_bytes"],
            desc["mla_width"], desc["mla_bytes"],
            desc.get("block_size", 0), desc.get("chunk_min_tokens", 1),
            int(desc.get("strict_chunk_multiple", 0)), desc["path"],
            int(desc.get("separate_object_groups", 1)),
            None if kvg_arr is None else kvg_arr.ctypes.data,
            desc["pool_bytes"], desc.get("max_num_batched_tokens", 0),
            int(desc.get("kda_codec", 0)), ctypes.byref(h))
        if rc != OK:
            raise OracleError(rc, "layout_init")
        self._h = h
        s = (ctypes.c_int64 * 15)()
        L.hkvref_layout_summary(h, s)
        self.summary = dict(zip(SUMMARY_FIELDS, [int(v) for v in s]))
        self.layers = []
        for l in range(self.summary["n_layers"]):
            o = (ctypes.c_int64 * 10)()
            L.hkvref_layer(h, l, o)
            self.layers.append(dict(zip(LAYER_FIELDS, [int(v) for v in o])))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and self._L is not None:
            self._L.hkvref_layout_free(h)
            self._h = None

    @property
    def G(self) -> int:
        return self.summary["n_kv_groups"]

    @property
    def O(self) -> int:
        return self.summary["n_obj_groups"]

    @property
    def k(self) -> int:
        return self.summary["blocks_per_chunk"]

    def obj_bytes(self, o: int) -> int:
        return self.summary["obj_bytes0"] if o == 0 else self.summary["obj_bytes1"]

    def _ids(self, block_ids) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int32))
        if ids.ndim != 3 or ids.shape[1:] != (self.G, self.k):
            raise ValueError(f"block_ids must be [n_chunks][{self.G}][{self.k}], got {ids.shape}")
        return ids

    def _check_buffers(self, pool: np.ndarray, objects) -> None:
        if not (isinstance(pool, np.ndarray) and pool.dtype == np.uint8
                and pool.flags.c_contiguous):
            raise TypeError("pool must be a C-contiguous uint8 numpy array")
        if pool.nbytes < self.summary["pool_bytes_used"]:
            raise ValueError("pool is smaller than the bytes the layout addresses")
        for objs in objects:
            for o, a in enumerate(objs):
                if a.nbytes < self.obj_bytes(o):
                    raise ValueError("object smaller than its object group's size")

    def _tokens(self, chunk_tokens, n):
        if chunk_tokens is None:
            return None, None
        t = np.ascontiguousarray(np.asarray(chunk_tokens, dtype=np.int32))
        if t.shape != (n,):
            raise ValueError(f"chunk_tokens must have shape ({n},)")
        return t, t.ctypes.data

    def store(self, pool: np.ndarray, block_ids, objects, chunk_tokens=None) -> None:
        ids = self._ids(block_ids)
        n = ids.shape[0] if ids.ndim else 0
        addrs = _ptr_array(objects, n, self.O)
        self._check_buffers(pool, objects)
        keep, tp = self._tokens(chunk_tokens, n)
        rc = self._L.hkvref_store_chunks(self._h, pool.ctypes.data, n, ids.ctypes.data, tp,
                                         addrs)
        if rc != OK:
            raise OracleError(rc, "store_chunks")

    def retrieve(self, pool: np.ndarray, block_ids, objects, chunk_tokens=None) -> None:
        ids = self._ids(block_ids)
        n = ids.shape[0] if ids.ndim else 0
        addrs = _ptr_array(objects, n, self.O)
        self._check_buffers(pool, objects)
        keep, tp = self._tokens(chunk_tokens, n)
        rc = self._L.hkvref_retrieve_chunks(self._h, pool.ctypes.data, n, ids.ctypes.data, tp,
                                            addrs)
        if rc != OK:
            raise OracleError(rc, "retrieve_chunks")

    def fingerprint(self) -> int:
        return int(self._L.hkvref_fingerprint(self._h))

    def codec_page(self, page, encode=True, layer=None):
        """One KDA page through the codec: a pool page (page bytes) to its
        object form, or (encode=False) back."""
        if layer is None:
            layer = next(l for l, L in enumerate(self.layers) if not L["is_mla"])
        L = self.layers[layer]
        src = np.ascontiguousarray(page, dtype=np.uint8)
        n_in, n_out = ((L["page_bytes"], L["obj_page_bytes"]) if encode
                       else (L["obj_page_bytes"], L["page_bytes"]))
        if src.size != n_in:
            raise ValueError(f"expected {n_in} bytes, got {src.size}")
        out = np.empty(n_out, np.uint8)
        rc = self._L.hkvref_codec_page(self._h, 1 if encode else 0, src.ctypes.data,
                                       out.ctypes.data)
        if rc != OK:
            raise OracleError(rc, "codec_page")
        return out

    def chunk_keys(self, tokens, hash_block_tokens=0, root=0, rank_tag=0):
        """(prefix hashes [n_tokens // h], keys [n_chunks][O]) as uint64 arrays."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        h = hash_block_tokens or self.summary["block_size"]
        n_fine = toks.size // h if h > 0 else 0
        n_chunks = toks.size // self.summary["chunk_tokens"]
        prefix = np.zeros(max(1, n_fine), dtype=np.uint64)
        keys = np.zeros((max(1, n_chunks), self.O), dtype=np.uint64)
        got = ctypes.c_int64()
        rc = self._L.hkvref_chunk_keys(self._h, toks.ctypes.data, toks.size, hash_block_tokens,
                                       root & (2**64 - 1), rank_tag & (2**64 - 1),
                                       prefix.ctypes.data, keys.ctypes.data, n_chunks,
                                       ctypes.byref(got))
        if rc != OK:
            raise OracleError(rc, "chunk_keys")
        return prefix[:n_fine], keys[:got.value]
