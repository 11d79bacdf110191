"""Object identity: the object-format fingerprint and chained prefix keys.

Pins of the oracle against what the pages fix:
- the i-th fine hash covers the whole prefix and nothing after it (vLLM
  hybrid KV-cache blog, section 6.3: each hash folds in the previous one);
- a chunk's hash is the hash of its last fine block (same section: a coarse
  block borrows its last fine sub-block's hash), so a request cut at a chunk
  boundary ends on that chunk's hash;
- hashing continues from a parent: hashing a suffix with root = the parent's
  last hash continues the parent's chain;
- keys separate object groups and parallel configurations (Mooncake K3 blog,
  vLLM x Mooncake);
- the fingerprint changes exactly when object bytes would mean something else
  (the recipes' Caveats: no sharing across backends or block sizes): it
  ignores the pool path, pool size, grouping and tuning, and moves with N,
  dtypes, layer pattern and object grouping.
Then the library against the oracle, bit for bit.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import retrieve_store_chunk_amd as hkv
import workloads as W


def small(path=0, sep=1, block_size=0, chunk_min=1, is_mla=(0, 0, 0, 1), mla_bytes=1,
          conv_dim=4, kvg=None):
    # 1 x 4 x 4 fp32 + (conv_dim, 3) bf16 state, 8 MLA values per token: N = 16
    return W._desc(list(is_mla), 1, 4, conv_dim, mla_bytes, path, 1 << 22,
                   block_size=block_size, chunk_min=chunk_min, kv_group_of_layer=kvg,
                   separate=sep, mla_width=8)


def tokens(seed, n):
    return np.random.default_rng(seed).integers(0, 2**31 - 1, n, dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------- pins
def test_fine_hash_covers_exactly_its_prefix():
    lay = oracle.Layout(small(chunk_min=48))   # N = 16, C = 48 (k = 3)
    h = 8
    t = tokens(1, 200)
    base, _ = lay.chunk_keys(t, h)
    assert base.size == 200 // h
    for pos in (0, 7, 8, 95, 96, 199):
        t2 = t.copy()
        t2[pos] ^= 0x5A5A
        got, _ = lay.chunk_keys(t2, h)
        first = pos // h                      # fine block holding the changed token
        assert np.array_equal(got[:first], base[:first])
        if first < base.size:
            assert np.all(got[first:] != base[first:])


def test_chunk_hash_is_its_last_fine_block_hash():
    lay = oracle.Layout(small(chunk_min=48))   # C = 48 tokens
    t = tokens(2, 48 * 5 + 20)
    for h in (1, 2, 4, 8, 16):
        fine, keys = lay.chunk_keys(t, h)
        assert keys.shape == (5, lay.O)        # whole chunks only
        for c in range(5):
            # a request cut at chunk c's end has chunk c as its last chunk and
            # ends its fine chain on the same hash
            cut_fine, cut_keys = lay.chunk_keys(t[: (c + 1) * 48], h)
            assert cut_fine[-1] == fine[(c + 1) * 48 // h - 1]
            assert np.array_equal(cut_keys[-1], keys[c])


def test_chain_continues_from_a_parent():
    lay = oracle.Layout(small(chunk_min=16))
    t = tokens(3, 160)
    for h in (4, 16):
        full, _ = lay.chunk_keys(t, h, root=77)
        a = 48
        head, _ = lay.chunk_keys(t[:a], h, root=77)
        tail, _ = lay.chunk_keys(t[a:], h, root=int(head[-1]))
        assert np.array_equal(np.concatenate([head, tail]), full)


def test_hash_depends_on_token_order_within_a_block():
    """The hash fingerprints the prefix, an ordered sequence: swapping two
    tokens of one hash block changes it."""
    lay = oracle.Layout(small())
    t = tokens(10, 64)
    t[3], t[4] = 11, 12
    base, kb = lay.chunk_keys(t)
    t[3], t[4] = 12, 11
    swapped, ks = lay.chunk_keys(t)
    assert base[0] != swapped[0] and np.all(kb != ks)


def test_shared_prefix_shares_keys():
    lay = oracle.Layout(small(chunk_min=32))
    a = tokens(4, 32 * 6)
    b = a.copy()
    b[32 * 4 + 3] += 1                          # diverge inside chunk 4
    _, ka = lay.chunk_keys(a)
    _, kb = lay.chunk_keys(b)
    assert np.array_equal(ka[:4], kb[:4])
    assert np.all(ka[4:] != kb[4:])


def test_keys_separate_groups_ranks_and_roots():
    lay = oracle.Layout(small())
    t = tokens(5, 64)
    _, k0 = lay.chunk_keys(t)
    assert lay.O == 2 and np.all(k0[:, 0] != k0[:, 1])
    _, k1 = lay.chunk_keys(t, rank_tag=(2 << 32) | 1)
    assert np.all(k0 != k1)
    _, k2 = lay.chunk_keys(t, root=1)
    assert np.all(k0 != k2)


def test_fingerprint_tracks_object_format_only():
    fp = lambda d: oracle.Layout(d).fingerprint()
    base = small()
    same = [small(path=1), dict(base, pool_bytes=1 << 23),
            small(kvg=[0, 1, 2, 3]), small(path=1, kvg=[0, 0, 0, 1])]
    for d in same:
        assert fp(d) == fp(base)
    # N matters even where it changes no page size (a model without MLA layers):
    # the k state pages of a chunk are snapshots at N-token boundaries
    assert fp(small(is_mla=(0, 0), block_size=16)) != fp(small(is_mla=(0, 0), block_size=32))
    differ = [small(block_size=32), small(chunk_min=17), small(mla_bytes=2),
              small(conv_dim=5), small(is_mla=(0, 0, 1, 1)), small(sep=0),
              small(is_mla=(0, 0, 0, 1, 0))]
    for d in differ:
        assert fp(d) != fp(base)
    # the workloads: path A and path B of the Kimi-Linear TP=1 shapes agree
    a = dict(W.make_config("kl_tp1").desc, path=0)
    assert fp(a) == fp(W.make_config("kl_tp1").desc)
    assert fp(W.make_config("kl_tp2").desc) != fp(W.make_config("kl_tp1").desc)


def test_bad_arguments():
    lay = oracle.Layout(small())
    with pytest.raises(oracle.OracleError):
        lay.chunk_keys(tokens(6, 32), hash_block_tokens=5)   # does not divide N = 16
    p, k = lay.chunk_keys(np.zeros(0, np.int32))
    assert p.size == 0 and k.shape[0] == 0
    p, k = lay.chunk_keys(tokens(7, 15))                     # shorter than one chunk
    assert p.size == 0 and k.shape[0] == 0


# ---------------------------------------------------------------- parity
@pytest.mark.parametrize("name", W.CONFIG_NAMES + W.EXTRA_CONFIG_NAMES)
def test_library_fingerprint_and_keys_match_oracle_on_workloads(name):
    d = W.make_config(name).desc
    ref, got = oracle.Layout(d), hkv.Layout(d)
    assert got.fingerprint() == ref.fingerprint()
    N = ref.summary["block_size"]
    t = tokens(8, 3 * ref.summary["chunk_tokens"] + N // 2)
    for h in (0, N // 2, 16):  # N is a multiple of 16 in every workload
        pr, kr = ref.chunk_keys(t, h, root=3, rank_tag=(8 << 32) | 5)
        pg, kg = got.chunk_keys(t, h, root=3, rank_tag=(8 << 32) | 5)
        assert np.array_equal(pr, pg) and np.array_equal(kr, kg)


@settings(max_examples=100, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.integers(0, 1), min_size=1, max_size=6), st.integers(0, 1), st.integers(0, 1),
       st.integers(1, 60), st.sampled_from([0, 1, 2, 4, 8, 16]), st.integers(0, 300),
       st.integers(0, 2**64 - 1), st.integers(0, 2**64 - 1))
def test_library_keys_match_oracle_on_random_inputs(is_mla, path, sep, cmin, h, n, root, tag):
    d = small(path=path, sep=sep, chunk_min=cmin, is_mla=is_mla)
    ref, got = oracle.Layout(d), hkv.Layout(d)
    assert got.fingerprint() == ref.fingerprint()
    t = tokens(n, n)
    pr, kr = ref.chunk_keys(t, h, root=root, rank_tag=tag)
    pg, kg = got.chunk_keys(t, h, root=root, rank_tag=tag)
    assert np.array_equal(pr, pg) and np.array_equal(kr, kg)


def test_library_rejects_what_the_oracle_rejects():
    d = small()
    got = hkv.Layout(d)
    assert hkv.status_of(got.chunk_keys, tokens(9, 32), 5) == hkv.HKV_E_ARG
    assert hkv.status_of(got.chunk_keys, tokens(9, 32), -4) == hkv.HKV_E_ARG
