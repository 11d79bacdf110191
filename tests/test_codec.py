"""The INT8 codec of inactive KDA checkpoints.

The Mooncake K3 blog (Compressed Checkpoint Storage) compresses inactive
recurrent states to INT8 with per-channel quantization parameters and keeps
the conv window at full precision.  It does not fix the axis or the rounding.
The readings, implemented by the oracle and the library, are:

- a channel is one row of head_dim fp32 values;
- s = (largest finite |x|) / 127;
- q = round-half-even(x / s), clamped to +-127, and 0 for non-finite x or s == 0;
- decoding gives q * s;
- a KDA page is the conv state, then the recurrent state.

Pins of the oracle (CPU), each a property rather than a retyped formula:
the round-off bound, the extremal code, exact lattices, the tie rule, zero
and non-finite rows, denormals, the verbatim conv part, object sizes, nulls,
the fingerprint and the rejected shapes.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads as W

H, D, CONV = 2, 16, 96   # the tiny workload's state: 2 x 16 x 16 fp32 + (96, 3) bf16
CONV_PART = CONV * 3 * 2
ROWS = H * D


def codec_desc(**kw):
    d = dict(W.make_config("tiny").desc, kda_codec=1)
    d.update(kw)
    return d


def pages_with_rows(lay, rows_fn, seed=0):
    """A pool whose KDA pages hold conv bytes + recurrent rows from rows_fn."""
    s = lay.summary
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 256, s["pool_bytes_used"], dtype=np.uint8)
    kda = [l for l, L in enumerate(lay.layers) if not L["is_mla"]]
    for b in range(s["num_blocks"]):
        for l in kda:
            L = lay.layers[l]
            base = L["pool_offset"] + b * L["stride"] + CONV_PART
            pool[base: base + ROWS * D * 4] = rows_fn(rng).astype("<f4").view(np.uint8).ravel()
    return pool


def store_one(lay, pool, block):
    """Store chunk 0 from blocks block, block + 1, ... (one per group and j)."""
    ids = (block + np.arange(lay.G * lay.k, dtype=np.int32)).reshape(1, lay.G, lay.k)
    objs = [[np.zeros(lay.obj_bytes(o), np.uint8) for o in range(lay.O)]]
    lay.store(pool, ids, objs)
    return ids, objs


def split_kda_page(lay, objs, layer):
    L = lay.layers[layer]
    page = objs[0][L["obj_group"]][L["obj_offset"]: L["obj_offset"] + L["obj_page_bytes"]]
    conv = page[:CONV_PART]
    codes = page[CONV_PART: CONV_PART + ROWS * D].view(np.int8).reshape(ROWS, D)
    scales = page[CONV_PART + ROWS * D:].view("<f4")
    return conv, codes, scales


def source_rows(lay, pool, layer, block):
    L = lay.layers[layer]
    base = L["pool_offset"] + block * L["stride"]
    page = pool[base: base + L["page_bytes"]]
    return page[:CONV_PART], page[CONV_PART:].view("<f4").reshape(ROWS, D)


def roundtrip(rows_fn, seed=0):
    lay = oracle.Layout(codec_desc())
    pool = pages_with_rows(lay, rows_fn, seed)
    ids, objs = store_one(lay, pool, 3)
    kda = [l for l, L in enumerate(lay.layers) if not L["is_mla"]]
    out = []
    fresh = np.zeros_like(pool)
    lay.retrieve(fresh, ids, objs)
    for l in kda:
        b = int(ids[0, lay.layers[l]["kv_group"], 0])
        conv_src, x = source_rows(lay, pool, l, b)
        conv_obj, q, s = split_kda_page(lay, objs, l)
        conv_back, y = source_rows(lay, fresh, l, b)
        out.append((x, q, s, y, conv_src, conv_obj, conv_back))
    return out


def test_object_page_is_conv_then_codes_then_scales():
    lay = oracle.Layout(codec_desc())
    for L in lay.layers:
        if L["is_mla"]:
            assert L["obj_page_bytes"] == L["page_bytes"]
        else:
            assert L["page_bytes"] == CONV_PART + ROWS * D * 4
            assert L["obj_page_bytes"] == CONV_PART + ROWS * D + ROWS * 4
    plain = oracle.Layout(W.make_config("tiny").desc)
    assert lay.summary["obj_bytes1"] == plain.summary["obj_bytes1"]      # MLA unchanged
    assert lay.summary["obj_bytes0"] < plain.summary["obj_bytes0"]


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.integers(0, 2**31 - 1), st.sampled_from([1e-30, 1e-3, 1.0, 7.5, 3e4, 1e30]))
def test_round_off_bound_and_extremal_code(seed, mag):
    """|x - q s| <= s / 2 for every finite value (plus fp32 rounding of the
    product), |q| <= 127, and the row's largest |x| encodes to +-127."""
    for x, q, s, y, conv_src, conv_obj, conv_back in roundtrip(
            lambda r: (r.standard_normal((ROWS, D)) * mag).astype(np.float32), seed):
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        amax = np.abs(x).max(axis=1)
        assert np.all(s >= 0)
        err = np.abs(x.astype(np.float64) - y.astype(np.float64))
        bound = s.astype(np.float64)[:, None] * (0.5 + 1e-6) + np.abs(x) * 2.0 ** -23
        assert np.all(err <= bound)
        top = np.argmax(np.abs(x), axis=1)
        rows = np.arange(ROWS)
        assert np.all(np.abs(q[rows, top]) == 127)
        assert np.all(np.sign(q[rows, top]) == np.sign(x[rows, top]))
        # scale = largest |x| / 127 to within one fp32 rounding
        assert np.allclose(s, amax / 127.0, rtol=2 ** -22, atol=0)
        # the conv window is kept verbatim
        assert np.array_equal(conv_src, conv_obj) and np.array_equal(conv_src, conv_back)


def test_power_of_two_lattice_round_trips_exactly():
    """Values k * 2^e with max |k| = 127: s = 2^e exactly, every x / s is the
    integer k, so decoding is exact."""
    def rows(r):
        k = r.integers(-127, 128, (ROWS, D)).astype(np.float32)
        k[:, 0] = 127.0 * np.where(r.random(ROWS) < 0.5, -1, 1)
        e = r.integers(-20, 20, (ROWS, 1)).astype(np.float32)
        return k * np.exp2(e)
    for x, q, s, y, *_ in roundtrip(rows, seed=3):
        assert np.array_equal(y, x)
        assert np.array_equal(q.astype(np.float32) * s[:, None], x)


def test_ties_round_half_to_even():
    """With s = 1 (largest |x| = 127) the codes of x = n + 1/2 go to the even
    neighbour: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.5 -> 0, 126.5 -> 126."""
    vals = np.array([127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 126.5, -1.5, 1.5, 4.5, 5.5, -3.5,
                     0.0, 6.0, -127.0, 64.5], dtype=np.float32)
    want = np.array([127, 2, 4, -2, 0, 0, 126, -2, 2, 4, 6, -4, 0, 6, -127, 64])
    for x, q, s, y, *_ in roundtrip(lambda r: np.tile(vals, (ROWS, 1))):
        assert np.all(s == 1.0)
        assert np.array_equal(q, np.tile(want, (ROWS, 1)))


def test_zero_and_non_finite_rows():
    def rows(r):
        x = (r.standard_normal((ROWS, D)) * 3).astype(np.float32)
        x[0] = 0.0                                   # an all-zero row
        x[1, 3], x[1, 7], x[1, 9] = np.nan, np.inf, -np.inf
        x[2] = np.nan                                # nothing finite
        x[3, :] = 0.0
        x[3, 5] = -0.0
        return x
    for x, q, s, y, *_ in roundtrip(rows):
        assert s[0] == 0 and not q[0].any() and not y[0].any()
        finite = np.isfinite(x[1])
        assert np.all(q[1][~finite] == 0)
        assert s[1] == np.float32(np.abs(x[1][finite]).max()) / np.float32(127)
        assert s[2] == 0 and not q[2].any()
        assert s[3] == 0 and not q[3].any()


def test_denormal_rows():
    """Subnormal fp32 states quantise by the same IEEE arithmetic: the round-off
    bound holds and the extremal code is +-127."""
    def rows(r):
        return (r.standard_normal((ROWS, D)) * 1e-39).astype(np.float32)
    for x, q, s, y, *_ in roundtrip(rows):
        assert np.any((np.abs(x) > 0) & (np.abs(x) < np.finfo(np.float32).tiny))
        err = np.abs(x.astype(np.float64) - y.astype(np.float64))
        assert np.all(err <= s.astype(np.float64)[:, None] * 0.5 + 2 ** -149)
        top = np.argmax(np.abs(x), axis=1)
        assert np.all(np.abs(q[np.arange(ROWS), top]) == 127)


def test_null_pages_and_mla_pages_under_the_codec():
    lay = oracle.Layout(codec_desc())
    pool = pages_with_rows(lay, lambda r: r.standard_normal((ROWS, D)).astype(np.float32))
    plain = oracle.Layout(W.make_config("tiny").desc)
    ids = np.array([[[5], [6], [7], [8]]], dtype=np.int32)
    ids[0, 1, 0] = oracle.NULL_BLOCK
    a = [[np.full(lay.obj_bytes(o), 9, np.uint8) for o in range(lay.O)]]
    b = [[np.full(plain.obj_bytes(o), 9, np.uint8) for o in range(plain.O)]]
    lay.store(pool, ids, a)
    plain.store(pool, ids, b)
    assert np.array_equal(a[0][1], b[0][1])                # MLA pages: opaque copies
    L = [L for L in lay.layers if L["kv_group"] == 1][0]   # the null KDA page
    assert not a[0][0][L["obj_offset"]: L["obj_offset"] + L["obj_page_bytes"]].any()
    before = pool.copy()
    lay.retrieve(pool, ids, a)                             # writes nothing for the null page
    Lp = lay.layers[[l for l, x in enumerate(lay.layers) if x["kv_group"] == 1][0]]
    lo = Lp["pool_offset"] + 6 * Lp["stride"]
    assert np.array_equal(pool[lo: lo + Lp["page_bytes"]], before[lo: lo + Lp["page_bytes"]])


def test_codec_changes_the_fingerprint_and_rejects_unsupported_shapes():
    assert oracle.Layout(codec_desc()).fingerprint() != \
        oracle.Layout(W.make_config("tiny").desc).fingerprint()
    for bad in (dict(kda_state_bytes=2), dict(kda_head_dim=48), dict(kda_head_dim=8),
                dict(conv_dim=5), dict(kda_codec=2)):
        with pytest.raises(oracle.OracleError) as e:
            oracle.Layout(codec_desc(**bad))
        assert e.value.status == oracle.E_ARG


def test_decode_of_objects_the_encoder_did_not_write():
    """Decoding is the fp32 product q * s for every code, -128 included; a NaN
    result is written as the default quiet NaN 0x7FC00000 whatever its
    operands' payloads, and finite products keep every bit (denormals too)."""
    lay = oracle.Layout(codec_desc())
    L = next(L for L in lay.layers if not L["is_mla"])
    obj = np.zeros(L["obj_page_bytes"], np.uint8)
    obj[:CONV_PART] = np.arange(CONV_PART) % 251
    codes = obj[CONV_PART: CONV_PART + ROWS * D].view(np.int8).reshape(ROWS, D)
    scales = obj[CONV_PART + ROWS * D:].view("<u4")
    codes[:] = np.arange(-128, 128, 256 // D, dtype=np.int16)[None, :D].astype(np.int8)
    codes[:, 1] = 0
    scales[0] = 0x7FC12345                           # NaN with a payload
    scales[1] = 0x7F800000                           # +inf: inf * 0 is NaN, inf * q is +-inf
    scales[2] = 0xFF812345                           # negative signalling-pattern NaN
    scales[3] = np.float32(-0.5).view("<u4")
    scales[4] = 0x00000003                           # a denormal scale
    page = lay.codec_page(obj, encode=False)
    assert np.array_equal(page[:CONV_PART], obj[:CONV_PART])
    y = page[CONV_PART:].view("<u4").reshape(ROWS, D)
    assert np.all(y[0] == 0x7FC00000) and np.all(y[2] == 0x7FC00000)
    assert y[1, 1] == 0x7FC00000
    q = codes[1].astype(np.float32)
    assert np.array_equal(y[1][q > 0], np.full((q > 0).sum(), 0x7F800000, np.uint32))
    assert np.array_equal(y[1][q < 0], np.full((q < 0).sum(), 0xFF800000, np.uint32))
    assert codes[3, 0] == -128
    assert np.array_equal(y[3].view(np.float32), codes[3].astype(np.float32) * np.float32(-0.5))
    want4 = (codes[4].astype(np.float64) * 3 * 2.0 ** -149).astype(np.float32)
    assert np.array_equal(y[4].view(np.float32), want4)

