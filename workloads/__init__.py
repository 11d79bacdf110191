"""Seeded synthetic inputs for chunk store/retrieve.

The oracle side and the HIP side both draw their inputs from here, and from
nowhere else.  The module holds none of the method's arithmetic: no page
sizes, offsets, block-size or chunk rules.  It holds only:

1. SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
   generators", OOPSLA 2014), used as a counter-based byte generator.  Word q
   of a buffer with seed s is ``mix64(s + (q + 1) * GAMMA)``, little-endian.
   Because any word can be computed from its index alone, a large pool can be
   filled on the GPU (``workloads.gpu_fill``) and any sampled range checked on
   the host.
2. Fisher-Yates permutations of block ids, drawn from a SplitMix64 stream.
3. The five workload descriptions: model shapes, pool sizes and request mix.
4. Planning of waves of whole requests, given the pool's block count and the
   number of block ids each chunk needs (both read back from a layout).
"""
from __future__ import annotations

import copy
import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK = (1 << 64) - 1

HERE = os.path.dirname(os.path.abspath(__file__))
FILL_LIB_PATH = os.path.join(HERE, "libhkvfill.so")


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def mix64_int(z: int) -> int:
    """SplitMix64's output function on one 64-bit integer (pure Python)."""
    z &= MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64's output function, vectorised over a uint64 array."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def words(seed: int, start: int, count: int) -> np.ndarray:
    """Words [start, start+count) of the counter-based stream with this seed."""
    q = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = np.uint64(seed & MASK) + q * np.uint64(GAMMA)
    return mix64(x)


def fill_bytes(seed: int, byte_start: int, nbytes: int) -> np.ndarray:
    """Bytes [byte_start, byte_start+nbytes) of the stream, as uint8."""
    if nbytes <= 0:
        return np.zeros(0, dtype=np.uint8)
    w0 = byte_start // 8
    w1 = (byte_start + nbytes + 7) // 8
    w = words(seed, w0, w1 - w0).astype("<u8", copy=False)
    b = w.view(np.uint8)
    off = byte_start - w0 * 8
    return b[off:off + nbytes].copy()


class Stream:
    """A sequential SplitMix64 stream (state += GAMMA; output mix64(state))."""

    def __init__(self, seed: int):
        self.state = seed & MASK

    def next(self) -> int:
        self.state = (self.state + GAMMA) & MASK
        return mix64_int(self.state)


def derive_seed(*parts: int) -> int:
    """A seed for a named sub-stream: folds the integer parts through mix64."""
    h = 0
    for p in parts:
        h = mix64_int((h + (p & MASK) * GAMMA + 0x2545F4914F6CDD1D) & MASK)
    return h


def permutation(seed: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of range(n) driven by a SplitMix64 stream: for i
    from n-1 down to 1, swap element i with element next() % (i+1)."""
    perm = list(range(n))
    s = Stream(seed)
    for i in range(n - 1, 0, -1):
        j = s.next() % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    return np.asarray(perm, dtype=np.int32)


# Sub-stream tags.
TAG_POOL, TAG_OBJ, TAG_STORE_IDS, TAG_RETRIEVE_IDS, TAG_REQUESTS, TAG_SHARED_IDS = 1, 2, 3, 4, 5, 6


# --------------------------------------------------------------------------
# GPU fill (same stream definition, for pools too large to copy from host)
# --------------------------------------------------------------------------
_fill_lib = None


def _load_fill():
    global _fill_lib
    if _fill_lib is None:
        if not os.path.exists(FILL_LIB_PATH):
            raise RuntimeError(f"{FILL_LIB_PATH} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (bind to torch's HIP runtime; see retrieve_store_chunk_amd)
        L = ctypes.CDLL(FILL_LIB_PATH)
        L.hkvfill_splitmix.restype = ctypes.c_int
        L.hkvfill_splitmix.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_void_p]
        L.hkvfill_rows.restype = ctypes.c_int
        L.hkvfill_rows.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        _fill_lib = L
    return _fill_lib


def gpu_fill(dev_ptr: int, nbytes: int, seed: int, byte_start: int = 0, stream: int = 0) -> None:
    """Fill nbytes of device memory at dev_ptr with stream bytes
    [byte_start, byte_start+nbytes) of `seed`.  byte_start must be a multiple
    of 8 and dev_ptr 8-byte aligned."""
    if nbytes == 0:
        return
    if byte_start % 8 or dev_ptr % 8:
        raise ValueError("gpu_fill needs 8-byte aligned start and pointer")
    rc = _load_fill().hkvfill_splitmix(dev_ptr, nbytes, seed & MASK, byte_start // 8, stream)
    if rc != 0:
        raise RuntimeError(f"gpu fill failed with HIP error {rc}")


ROW_ZEROS = 1 << 63


def gpu_fill_rows(buf, rows: np.ndarray, stream: int = 0) -> None:
    """Rows of streams at given places in a device uint8 tensor `buf`: rows is
    an array [n][4] of (byte offset, seed, first word, word count); a count
    with ROW_ZEROS set writes that many zero words instead.  Rows of one call
    must not overlap (they run in parallel).  Every row is checked to lie
    inside the buffer before the launch."""
    import torch
    rows = np.ascontiguousarray(rows, dtype=np.uint64).reshape(-1, 4)
    if rows.shape[0] == 0:
        return
    off = rows[:, 0]
    n_words = rows[:, 3] & np.uint64(ROW_ZEROS - 1)
    if (off % np.uint64(8)).any():
        raise ValueError("row offsets must be multiples of 8")
    if (off + n_words * np.uint64(8) > np.uint64(buf.numel())).any():
        raise ValueError("a row ends past the buffer")
    if buf.data_ptr() % 8:
        raise ValueError("buffer must be 8-byte aligned")
    # one launch covers at most 2^32 - 1 work items (256 per 64 KiB tile)
    tiles = max(1, (int(n_words.max()) + 8191) // 8192)
    per_launch = max(1, (0xFFFFFFFF // 256) // tiles)
    for lo in range(0, rows.shape[0], per_launch):
        part = rows[lo:lo + per_launch]
        dev_rows = torch.from_numpy(np.ascontiguousarray(part).view(np.int64)).to(buf.device)
        rc = _load_fill().hkvfill_rows(buf.data_ptr(), buf.numel(), dev_rows.data_ptr(),
                                       part.shape[0], int(n_words.max()), stream)
        if rc != 0:
            raise RuntimeError(f"gpu row fill failed with HIP error {rc}")
        # the table must outlive the launch that reads it
        if stream:
            torch.cuda.ExternalStream(stream).synchronize()
        else:
            torch.cuda.synchronize()
        del dev_rows
    if stream:
        torch.cuda.ExternalStream(stream).synchronize()
    else:
        torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
GIB = 1 << 30
MIB = 1 << 20


def kkkm_pattern(n_layers: int, tail_mla: int = 0) -> list:
    """Layer types for the "three KDA layers then one MLA layer" pattern
    (1 = MLA), with `tail_mla` extra MLA layers at the end.  Kimi-Linear's 27
    layers: kkkm_pattern(24) + [0, 0, 1]; K3's 93: kkkm_pattern(92, 1)."""
    return [1 if i % 4 == 3 else 0 for i in range(n_layers)] + [1] * tail_mla


KIMI_LINEAR_27 = kkkm_pattern(24) + [0, 0, 1]
K3_93 = kkkm_pattern(92, tail_mla=1)


def _desc(is_mla, heads, head_dim, conv_dim, mla_bytes, path, pool_bytes, block_size=0,
          chunk_min=1, kv_group_of_layer=None, separate=1, state_bytes=4, conv_kernel=4,
          conv_bytes=2, mla_width=576, strict=0, max_batched=0, kda_codec=0) -> dict:
    return dict(is_mla=list(is_mla), kda_heads=heads, kda_head_dim=head_dim,
                kda_state_bytes=state_bytes, conv_dim=conv_dim, conv_kernel=conv_kernel,
                conv_bytes=conv_bytes, mla_width=mla_width, mla_bytes=mla_bytes,
                block_size=block_size, chunk_min_tokens=chunk_min, strict_chunk_multiple=strict,
                path=path, separate_object_groups=separate,
                kv_group_of_layer=kv_group_of_layer, pool_bytes=pool_bytes,
                max_num_batched_tokens=max_batched, kda_codec=kda_codec)


@dataclass
class Phase:
    op: str                       # "store" or "retrieve"
    chunks: list                  # [(request, chunk_index)] in request then chunk order
    prefilled_objects: bool = False  # retrieve of objects that no store in this run made
    # KDA snapshots exist only at every snapshot_every-th block boundary of a
    # request (a scheduler step spanning several blocks snapshots only its
    # last one); other KDA block-table entries are null.
    snapshot_every: int = 1
    # (request, chunk) -> valid tokens of a partial chunk (a tail); KDA blocks
    # not completed inside it and MLA blocks past its last token are null.
    tail_tokens: dict = field(default_factory=dict)


@dataclass
class Config:
    name: str
    title: str
    desc: dict
    requests: list                # chunks per request
    phases: list                  # [Phase]
    seed: int
    shared_permutation: bool = False  # all phases draw ids from one permutation
    notes: str = ""
    extra: dict = field(default_factory=dict)
    shapes: str = ""              # short name of the shapes, for the benchmark's metric line


def _all_chunks(requests, first=None):
    out = []
    for r, n in enumerate(requests):
        m = n if first is None else min(first, n)
        out += [(r, c) for c in range(m)]
    return out


def _tiny_requests(seed: int) -> list:
    s = Stream(derive_seed(seed, TAG_REQUESTS))
    return [3 + s.next() % 3 for _ in range(4)]


SHAPES = {
    "tiny": "tiny 4-layer shapes",
    "kl_tp2": "Kimi-Linear TP=2 rank shapes",
    "kl_tp1": "Kimi-Linear shapes",
    "k3_tp8": "K3-shaped TP=8 rank",
    "long_ctx": "Kimi-Linear shapes, long context",
    "kl_tp1_host": "Kimi-Linear shapes, pinned host objects",
    "k3_tp8_holes": "K3-shaped TP=8 rank, KDA snapshots every 4th block",
    "kl_tp1_tails": "Kimi-Linear shapes, partial tails",
    "kl_tp1_host_duplex": "Kimi-Linear shapes, pinned host objects, store and retrieve at once",
    "kl_tp1_int8": "Kimi-Linear shapes, INT8 KDA objects",
    "kl_tp1_int8_host": "Kimi-Linear shapes, INT8 KDA objects in pinned host memory",
}


def make_config(name: str) -> Config:
    """A workload at full size: the five of the benchmark's configurations
    (CONFIG_NAMES) and the further ones (EXTRA_CONFIG_NAMES)."""
    cfg = _make_config(name)
    cfg.shapes = SHAPES[name]
    return cfg


def _make_config(name: str) -> Config:
    if name == "tiny":
        seed = 0x48B0001
        req = _tiny_requests(seed)
        # 4 layers KKKM; 2 heads x 16 x 16 fp32 + (96, 3) bf16; bf16 MLA;
        # path A pool of 64 blocks of the unified page (64 x 16 x 576 x 2 B).
        desc = _desc([0, 0, 0, 1], 2, 16, 96, 2, 0, 64 * 16 * 576 * 2)
        return Config(name, "Tiny: 4 layers (3 KDA + 1 MLA), path A, 64 blocks", desc, req,
                      [Phase("store", _all_chunks(req)), Phase("retrieve", _all_chunks(req))],
                      seed)
    if name == "kl_tp2":
        seed = 0x48B0002
        req = [8] * 64
        desc = _desc(KIMI_LINEAR_27, 16, 128, 6144, 2, 0, 16 * GIB)
        return Config(name, "Kimi-Linear-48B-A3B, one TP=2 rank, path A, 16 GiB pool", desc,
                      req, [Phase("store", _all_chunks(req)),
                            Phase("retrieve", _all_chunks(req))], seed)
    if name == "kl_tp1":
        seed = 0x48B0003
        req = [8] * 128
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB)
        return Config(name, "Kimi-Linear full state (TP=1), path B, 64 GiB pool", desc, req,
                      [Phase("store", _all_chunks(req)),
                       Phase("retrieve", _all_chunks(req, first=4))], seed,
                      notes="128 requests of 16k tokens = 8 whole chunks each; the retrieve "
                            "hits the first 4 chunks of every request (50% prefix hits)")
    if name == "k3_tp8":
        seed = 0x48B0004
        req = [4] * 256
        desc = _desc(K3_93, 6, 128, 2304, 1, 0, 24 * GIB, block_size=768, chunk_min=1500)
        return Config(name, "K3-shaped TP=8 rank, path A, fp8 MLA, N=768, chunk min 1500, "
                      "24 GiB pool", desc, req,
                      [Phase("store", _all_chunks(req)), Phase("retrieve", _all_chunks(req))],
                      seed)
    if name == "long_ctx":
        seed = 0x48B0005
        # 1,000,000 tokens = 529 whole chunks of 1888 + a 1,248-token partial
        # one; a 2,048-token request = one whole chunk + a 160-token tail
        prefix_tokens, request_tokens, chunk = 1_000_000, 2048, 1888
        n_prefix = -(-prefix_tokens // chunk)
        req = [n_prefix] + [2] * 512
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 100 * GIB)
        prefix_tail = {(0, n_prefix - 1): prefix_tokens - (n_prefix - 1) * chunk}
        tails = {(r, 1): request_tokens - chunk for r in range(1, 513)}
        return Config(name, "Long context: 1,000,000-token prefix retrieve (529 whole chunks "
                      "+ a 1,248-token tail) + 512 stores of 2,048-token requests, path B, "
                      "100 GiB pool", desc, req,
                      [Phase("retrieve", [(0, c) for c in range(n_prefix)],
                             prefilled_objects=True, tail_tokens=prefix_tail),
                       Phase("store", [(r, c) for r in range(1, 513) for c in range(2)],
                             tail_tokens=tails)],
                      seed, shared_permutation=True,
                      notes="the prefix is 529 whole chunks of 1888 tokens and a last chunk of "
                            "1,248 tokens (MLA rows only: its KDA block is not complete); each "
                            "2,048-token request stores one whole chunk and a 160-token tail")
    if name == "kl_tp1_host":
        seed = 0x48B0006
        req = [8] * 16
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB)
        return Config(name, "Kimi-Linear full state (TP=1), path B, chunk objects in pinned "
                      "host memory", desc, req,
                      [Phase("store", _all_chunks(req)),
                       Phase("retrieve", _all_chunks(req, first=4))], seed,
                      notes="16 requests x 8 chunks stored to host objects (7.5 GB pinned), "
                            "the first 4 chunks of each retrieved from them",
                      extra={"objects": "host"})
    if name == "k3_tp8_holes":
        seed = 0x48B0007
        req = [4] * 256
        desc = _desc(K3_93, 6, 128, 2304, 1, 0, 24 * GIB, block_size=768, chunk_min=1500,
                     max_batched=4 * 768)
        every = 4  # a 4N token budget: each step advances 4 blocks, snapshots its last
        return Config(name, "K3-shaped TP=8 rank, token budget 4N: KDA snapshots at every "
                      "4th block only", desc, req,
                      [Phase("store", _all_chunks(req), snapshot_every=every),
                       Phase("retrieve", _all_chunks(req), snapshot_every=every)], seed,
                      notes="the K3 workload with a scheduler budget of 4N (allowed with "
                            "separate object groups): 3 of every 4 KDA block-table entries "
                            "are null")
    if name == "kl_tp1_tails":
        seed = 0x48B0008
        req = [2] * 256
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB)
        tails = {(r, 1): 2048 - 1888 for r in range(256)}
        return Config(name, "Kimi-Linear TP=1, path B: 256 requests of 2048 tokens = one "
                      "whole chunk + a 160-token partial tail", desc, req,
                      [Phase("store", _all_chunks(req), tail_tokens=tails),
                       Phase("retrieve", _all_chunks(req), tail_tokens=tails)], seed,
                      notes="each request stores its whole first chunk and a partial second "
                            "chunk (160 MLA rows, no KDA snapshot: its block is not complete)")
    if name == "kl_tp1_host_duplex":
        seed = 0x48B000A
        req = [8] * 16
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB)
        return Config(name, "Kimi-Linear full state (TP=1), path B, host objects: a store "
                      "(kernels) and a retrieve (DMA) at the same time on two streams", desc, req,
                      [Phase("retrieve", [(r, c) for r in range(8) for c in range(8)],
                             prefilled_objects=True),
                       Phase("store", [(r, c) for r in range(8, 16) for c in range(8)])],
                      seed, shared_permutation=True,
                      notes="requests 0-7 (64 chunks) are retrieved from pinned host objects "
                            "while requests 8-15 (64 chunks) are stored to them, on two streams; "
                            "the phases draw their block ids from one permutation, so they "
                            "touch different blocks",
                      extra={"objects": "host", "duplex": True, "retrieve_engine": "dma"})
    if name == "kl_tp1_int8":
        seed = 0x48B0009
        req = [8] * 128
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB, kda_codec=1)
        return Config(name, "Kimi-Linear full state (TP=1), path B, KDA recurrent state "
                      "stored as per-row INT8", desc, req,
                      [Phase("store", _all_chunks(req)),
                       Phase("retrieve", _all_chunks(req, first=4))], seed,
                      notes="the Kimi-Linear TP=1 workload with the INT8 codec of KDA "
                            "checkpoints: 3.5x smaller KDA objects, quantised on store and "
                            "dequantised on retrieve in the same pass")
    if name == "kl_tp1_int8_host":
        seed = 0x48B000B
        req = [8] * 16
        desc = _desc(KIMI_LINEAR_27, 32, 128, 12288, 2, 1, 64 * GIB, kda_codec=1)
        return Config(name, "Kimi-Linear full state (TP=1), path B, INT8 KDA objects in "
                      "pinned host memory", desc, req,
                      [Phase("store", _all_chunks(req)),
                       Phase("retrieve", _all_chunks(req, first=4))], seed,
                      notes="the host-object workload with the INT8 codec: 16 requests x 8 "
                            "chunks stored to host objects (2.2 GB pinned instead of 7.5 GB), "
                            "the first 4 chunks of each retrieved from them",
                      extra={"objects": "host"})
    raise KeyError(name)


CONFIG_NAMES = ("tiny", "kl_tp2", "kl_tp1", "k3_tp8", "long_ctx")
# Further workloads beyond the five above.
EXTRA_CONFIG_NAMES = ("kl_tp1_host", "k3_tp8_holes", "kl_tp1_tails", "kl_tp1_int8",
                      "kl_tp1_host_duplex", "kl_tp1_int8_host")


def make_small_config(name: str) -> Config:
    """The same page shapes with a smaller pool and fewer requests, so the
    oracle finishes in seconds; still several waves, several tiles per page
    and ragged sub-tiles."""
    cfg = copy.deepcopy(make_config(name))
    if name == "tiny":
        return cfg
    if name == "kl_tp2":
        cfg.desc["pool_bytes"] = 512 * MIB
        cfg.requests = [3] * 6
        cfg.phases = [Phase("store", _all_chunks(cfg.requests)),
                      Phase("retrieve", _all_chunks(cfg.requests))]
    elif name == "kl_tp1":
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [4] * 5
        cfg.phases = [Phase("store", _all_chunks(cfg.requests)),
                      Phase("retrieve", _all_chunks(cfg.requests, first=2))]
    elif name == "k3_tp8":
        cfg.desc["pool_bytes"] = 512 * MIB
        cfg.requests = [2] * 7
        cfg.phases = [Phase("store", _all_chunks(cfg.requests)),
                      Phase("retrieve", _all_chunks(cfg.requests))]
    elif name == "kl_tp1_int8":
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [4] * 5
        cfg.phases = [Phase("store", _all_chunks(cfg.requests)),
                      Phase("retrieve", _all_chunks(cfg.requests, first=2))]
    elif name == "kl_tp1_host_duplex":
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [2] * 4
        cfg.phases = [Phase("retrieve", [(r, c) for r in range(2) for c in range(2)],
                            prefilled_objects=True),
                      Phase("store", [(r, c) for r in range(2, 4) for c in range(2)])]
    elif name in ("kl_tp1_host", "kl_tp1_int8_host"):
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [4] * 3
        cfg.phases = [Phase("store", _all_chunks(cfg.requests)),
                      Phase("retrieve", _all_chunks(cfg.requests, first=2))]
    elif name == "k3_tp8_holes":
        cfg.desc["pool_bytes"] = 512 * MIB
        cfg.requests = [4] * 3
        cfg.phases = [Phase("store", _all_chunks(cfg.requests), snapshot_every=4),
                      Phase("retrieve", _all_chunks(cfg.requests), snapshot_every=4)]
    elif name == "kl_tp1_tails":
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [2] * 8
        tails = {(r, 1): 160 for r in range(8)}
        cfg.phases = [Phase("store", _all_chunks(cfg.requests), tail_tokens=tails),
                      Phase("retrieve", _all_chunks(cfg.requests), tail_tokens=tails)]
    elif name == "long_ctx":
        cfg.desc["pool_bytes"] = 1 * GIB
        cfg.requests = [6] + [2] * 4
        cfg.phases = [Phase("retrieve", [(0, c) for c in range(6)], prefilled_objects=True,
                            tail_tokens={(0, 5): 1248}),
                      Phase("store", [(r, c) for r in range(1, 5) for c in range(2)],
                            tail_tokens={(r, 1): 160 for r in range(1, 5)})]
    cfg.name = name + "_small"
    return cfg


# --------------------------------------------------------------------------
# Waves and block tables
# --------------------------------------------------------------------------
NULL_BLOCK = -1


@dataclass
class Wave:
    op: str
    chunks: list          # [(request, chunk_index)]
    ids: np.ndarray       # int32 [n_chunks][G][k] (NULL_BLOCK for a missing page)
    pool_seed: int | None  # store waves: the pool is (re)filled with this seed first
    prefilled_objects: bool = False
    chunk_tokens: np.ndarray | None = None  # int32 [n_chunks] valid tokens; None: all whole


def object_seed(cfg: Config, request: int, chunk: int) -> int:
    return derive_seed(cfg.seed, TAG_OBJ, request, chunk)


def _split_waves(chunks, max_chunks: int):
    """Greedy waves of whole requests, each at most max_chunks chunks."""
    if max_chunks < 1:
        raise ValueError("the pool cannot hold one chunk's blocks")
    waves, cur, cur_req = [], [], None
    by_req = {}
    for rc in chunks:
        by_req.setdefault(rc[0], []).append(rc)
    for r in sorted(by_req):
        group = by_req[r]
        if len(group) > max_chunks:
            raise ValueError("a request has more chunks than the pool holds at once")
        if len(cur) + len(group) > max_chunks:
            waves.append(cur)
            cur = []
        cur = cur + group
        cur_req = r
    if cur:
        waves.append(cur)
    del cur_req
    return waves


def plan_waves(cfg: Config, num_blocks: int, n_kv_groups: int, blocks_per_chunk: int,
               kda_groups=(), block_tokens: int = 0, chunk_tokens: int = 0) -> list:
    """Block tables for every wave.  Ids are assigned from a Fisher-Yates
    permutation of [0, num_blocks) in request order, chunk order, KV-group
    order, then block order; every wave of a phase draws a fresh permutation
    (fresh, fragmented ids), or all phases share one permutation when the
    config says so.  Phases with holes or tails also need the KV groups of
    KDA layers, N and the chunk size (read back from a layout) to null the
    missing entries."""
    ids_per_chunk = n_kv_groups * blocks_per_chunk
    max_chunks = num_blocks // ids_per_chunk
    waves = []
    shared = None
    shared_pos = 0
    if cfg.shared_permutation:
        shared = permutation(derive_seed(cfg.seed, TAG_SHARED_IDS), num_blocks)
    for pi, ph in enumerate(cfg.phases):
        for wi, chunks in enumerate(_split_waves(ph.chunks, max_chunks)):
            need = len(chunks) * ids_per_chunk
            if shared is not None:
                if shared_pos + need > num_blocks:
                    raise ValueError("phases sharing one permutation do not fit the pool")
                flat = shared[shared_pos:shared_pos + need]
                shared_pos += need
            else:
                tag = TAG_STORE_IDS if ph.op == "store" else TAG_RETRIEVE_IDS
                flat = permutation(derive_seed(cfg.seed, tag, pi, wi), num_blocks)[:need]
            ids = flat.reshape(len(chunks), n_kv_groups, blocks_per_chunk).copy()
            toks = None
            if ph.snapshot_every > 1 or ph.tail_tokens:
                if not block_tokens or not chunk_tokens:
                    raise ValueError("holes and tails need the block and chunk sizes")
                toks = np.full(len(chunks), chunk_tokens, dtype=np.int32)
                for n, (r, c) in enumerate(chunks):
                    t = ph.tail_tokens.get((r, c), chunk_tokens)
                    toks[n] = t
                    for j in range(blocks_per_chunk):
                        b = c * blocks_per_chunk + j           # block index in the request
                        complete = (j + 1) * block_tokens <= t  # block ends inside the chunk
                        snap = complete and (b + 1) % ph.snapshot_every == 0
                        for g in range(n_kv_groups):
                            if g in kda_groups:
                                if not snap:
                                    ids[n, g, j] = NULL_BLOCK
                            elif j * block_tokens >= t:         # MLA block past the tail
                                ids[n, g, j] = NULL_BLOCK
            pool_seed = None
            if ph.op == "store" and not cfg.shared_permutation:
                pool_seed = derive_seed(cfg.seed, TAG_POOL, pi, wi)
            waves.append(Wave(ph.op, chunks, ids, pool_seed, ph.prefilled_objects, toks))
    return waves


def initial_pool_seed(cfg: Config) -> int:
    return derive_seed(cfg.seed, TAG_POOL, 0xFFFF)
