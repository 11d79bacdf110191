"""Properties every layout and every store/retrieve must satisfy.

These are statements about the result, not a second copy of the oracle's
formulas: a region either coincides with another or is disjoint from it,
pages of a group tile a block, a copy round-trips, a retrieve writes exactly
as many bytes as the pages it addresses.  Each names the passage it comes
from.
"""
from __future__ import annotations

import numpy as np


def group_members(layers):
    groups = {}
    for l, L in enumerate(layers):
        groups.setdefault(L["kv_group"], []).append(l)
    return groups


def check_path_a(summary, layers, pool_bytes):
    """vLLM hybrid KV-cache blog, section 3.1: every layer uses one page size
    (the largest page; smaller pages padded), tensors of page_size x
    num_blocks bytes are each shared by layers of different groups, and a
    block id sits at block_id x page_size inside every tensor."""
    P = summary["unified_page_bytes"]
    nb = summary["num_blocks"]
    assert P == max(L["page_bytes"] for L in layers)
    for L in layers:
        assert L["reserved_bytes"] == P and L["stride"] == P
        assert L["page_bytes"] <= P
    regions = {}
    for l, L in enumerate(layers):
        lo, hi = L["pool_offset"], L["pool_offset"] + nb * P
        assert 0 <= lo and hi <= summary["pool_bytes_used"] <= pool_bytes
        regions.setdefault((lo, hi), []).append(l)
    spans = sorted(regions)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0, "tensors must coincide or be disjoint"
    for members in regions.values():
        gs = [layers[l]["kv_group"] for l in members]
        assert len(set(gs)) == len(gs), "a tensor is shared only by layers of different groups"
    sizes = [len(m) for m in group_members(layers).values()]
    assert summary["n_slabs"] == len(regions) == max(sizes)
    assert summary["pool_bytes_used"] == len(regions) * nb * P
    assert (nb + 1) * len(regions) * P > pool_bytes, "num_blocks is the most that fits"


def check_path_b(summary, layers, pool_bytes):
    """vLLM hybrid KV-cache blog, section 3.2: within a group the layers'
    real pages follow one another (a running byte offset, model order); the
    block stride is the largest group total; num_blocks = available //
    block_stride."""
    S = summary["block_stride"]
    nb = summary["num_blocks"]
    totals = []
    for g, members in sorted(group_members(layers).items()):
        end = 0
        for l in members:  # model order
            L = layers[l]
            assert L["pool_offset"] == end, "pages of a group are packed in model order"
            assert L["reserved_bytes"] == L["page_bytes"]
            assert L["stride"] == S
            end += L["page_bytes"]
        totals.append(end)
    assert S == max(totals)
    assert nb * S == summary["pool_bytes_used"] <= pool_bytes < (nb + 1) * S


def check_objects(summary, layers):
    """"Hybrid Attention Models", Object-group separation: separated, the KDA
    layers and the full-attention layers are different objects; the byte
    layout inside an object (layer-major in model order, then block) is this
    library's reading."""
    k = summary["blocks_per_chunk"]
    O = summary["n_obj_groups"]
    kinds = {L["is_mla"] for L in layers}
    obj_bytes = [summary["obj_bytes0"], summary["obj_bytes1"]]
    if O == 2:
        assert kinds == {0, 1}
        for L in layers:
            assert L["obj_group"] == L["is_mla"]
    for o in range(O):
        end = 0
        for L in layers:
            if L["obj_group"] != o:
                continue
            assert L["obj_offset"] == end
            end += k * L["page_bytes"]
        assert end == obj_bytes[o]
    if O == 1:
        assert obj_bytes[1] == 0


def check_live_pages_disjoint(summary, layers):
    """With one shared block-id space (vLLM hybrid KV-cache blog, sections
    3.1 and 3.2) a block belongs to one group at a time: the pages of one
    group never overlap across blocks, and the pages of different blocks
    never overlap whatever groups own them.  Checked over every block."""
    nb = summary["num_blocks"]
    used = summary["pool_bytes_used"]
    per_group = {}
    cross = np.zeros(used, dtype=np.int32)
    for b in range(nb):
        mask = np.zeros(used, dtype=bool)
        for l, L in enumerate(layers):
            lo = L["pool_offset"] + b * L["stride"]
            hi = lo + L["page_bytes"]
            assert 0 <= lo and hi <= used
            mask[lo:hi] = True
            cnt = per_group.setdefault(L["kv_group"], np.zeros(used, dtype=np.int32))
            cnt[lo:hi] += 1
        cross += mask
    assert cross.max(initial=0) <= 1
    for cnt in per_group.values():
        assert cnt.max(initial=0) <= 1


def layer_views(layers, num_blocks, pool: np.ndarray):
    """Each layer's logical view of the one byte backing: (num_blocks,
    page_bytes) rows at its (offset, stride), the way the blog's section 3.2
    cuts views with as_strided and section 4.2 views a KDA page as
    (num_blocks, 1, 1, page_size_bytes)."""
    views = []
    for L in layers:
        v = np.lib.stride_tricks.as_strided(pool[L["pool_offset"]:],
                                            shape=(num_blocks, L["page_bytes"]),
                                            strides=(L["stride"], 1), writeable=False)
        views.append(v)
    return views


def objects_by_views(summary, layers, pool: np.ndarray, ids: np.ndarray):
    """Objects as concatenations of gathered view rows: object o of chunk c
    is, for each of its layers in model order, the rows of that layer's view
    at the chunk's block ids of the layer's group."""
    views = layer_views(layers, summary["num_blocks"], pool)
    out = []
    for c in range(ids.shape[0]):
        per_o = []
        for o in range(summary["n_obj_groups"]):
            parts = [views[l][ids[c, L["kv_group"], :]].reshape(-1)
                     for l, L in enumerate(layers) if L["obj_group"] == o]
            per_o.append(np.concatenate(parts) if parts else np.zeros(0, np.uint8))
        out.append(per_o)
    return out


def payload_bytes(summary, n_chunks: int) -> int:
    return n_chunks * (summary["obj_bytes0"] + summary["obj_bytes1"])
