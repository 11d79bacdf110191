"""The seeded input generators: the vectorised SplitMix64 equals its
definition, ranges are consistent, permutations are permutations, and the
wave plans respect the pool."""
import numpy as np
import pytest

import oracle
import workloads as W


def test_vectorised_splitmix_equals_definition():
    for seed in (0, 1, 0x48B0003, 2**64 - 1):
        s = W.Stream(seed)
        seq = [s.next() for _ in range(64)]
        assert W.words(seed, 0, 64).tolist() == seq
        assert W.words(seed, 10, 5).tolist() == seq[10:15]


def test_fill_bytes_is_little_endian_words_and_range_consistent():
    seed = 12345
    full = W.fill_bytes(seed, 0, 4096)
    w = W.words(seed, 0, 512)
    assert np.array_equal(full, w.astype("<u8").view(np.uint8))
    for start, n in [(0, 1), (3, 17), (8, 8), (1000, 1001), (4095, 1)]:
        assert np.array_equal(W.fill_bytes(seed, start, n), full[start:start + n])


def test_permutation_is_a_permutation_and_seeded():
    for n in (1, 2, 7, 64, 4513):
        p = W.permutation(99, n)
        assert sorted(p.tolist()) == list(range(n))
    assert np.array_equal(W.permutation(5, 100), W.permutation(5, 100))
    assert not np.array_equal(W.permutation(5, 100), W.permutation(6, 100))


def test_layer_patterns():
    assert len(W.KIMI_LINEAR_27) == 27 and sum(W.KIMI_LINEAR_27) == 7
    assert [i for i, m in enumerate(W.KIMI_LINEAR_27) if m] == [3, 7, 11, 15, 19, 23, 26]
    assert len(W.K3_93) == 93 and sum(W.K3_93) == 24 and W.K3_93[-2:] == [1, 1]


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
@pytest.mark.parametrize("small", [False, True])
def test_wave_plans_fit_the_pool(name, small):
    cfg = W.make_small_config(name) if small else W.make_config(name)
    lay = oracle.Layout(cfg.desc)
    s = lay.summary
    waves = _plan(cfg, lay)
    seen_store = set()
    for wv in waves:
        assert wv.ids.shape == (len(wv.chunks), lay.G, lay.k)
        flat = wv.ids.reshape(-1)
        flat = flat[flat != W.NULL_BLOCK]  # tails: no KDA snapshot for an incomplete block
        assert flat.min() >= 0 and flat.max() < s["num_blocks"]
        assert len(set(flat.tolist())) == flat.size  # unique within a wave
        reqs = sorted({r for r, _ in wv.chunks})
        for r in reqs:  # whole requests per wave
            in_wave = [c for rr, c in wv.chunks if rr == r]
            in_phase = [c for ph in cfg.phases if ph.op == wv.op
                        for rr, c in ph.chunks if rr == r]
            assert in_wave == in_phase
        if wv.op == "store":
            seen_store.update(wv.chunks)
    for ph in cfg.phases:
        if ph.op == "retrieve" and not ph.prefilled_objects:
            assert set(ph.chunks) <= seen_store
    if cfg.shared_permutation:
        allids = np.concatenate([wv.ids.reshape(-1) for wv in waves])
        allids = allids[allids != W.NULL_BLOCK]
        assert len(set(allids.tolist())) == allids.size


def _plan(cfg, lay):
    s = lay.summary
    kda = {L["kv_group"] for L in lay.layers if not L["is_mla"]}
    return W.plan_waves(cfg, s["num_blocks"], lay.G, lay.k, kda, s["block_size"],
                        s["chunk_tokens"])


def test_long_context_prefix_and_tails():
    """1,000,000 tokens are 529 whole chunks of 1888 and a 1,248-token one;
    a 2,048-token request is one whole chunk and a 160-token tail."""
    cfg = W.make_config("long_ctx")
    lay = oracle.Layout(cfg.desc)
    ret, st = _plan(cfg, lay)
    assert ret.op == "retrieve" and len(ret.chunks) == 530
    assert int(ret.chunk_tokens.sum()) == 1_000_000
    assert st.op == "store" and len(st.chunks) == 1024
    assert int(st.chunk_tokens.sum()) == 512 * 2048
    kda = [L["kv_group"] for L in lay.layers if not L["is_mla"]]
    assert (ret.ids[-1, sorted(set(kda)), :] == W.NULL_BLOCK).all()


def test_full_config_wave_counts():
    expect = {"kl_tp2": (1, 1), "kl_tp1": (1, 1), "k3_tp8": (4, 4), "long_ctx": (1, 1)}
    for name, (ns, nr) in expect.items():
        cfg = W.make_config(name)
        lay = oracle.Layout(cfg.desc)
        waves = _plan(cfg, lay)
        assert sum(w.op == "store" for w in waves) == ns
        assert sum(w.op == "retrieve" for w in waves) == nr
    cfg = W.make_config("k3_tp8")
    lay = oracle.Layout(cfg.desc)
    waves = W.plan_waves(cfg, lay.summary["num_blocks"], lay.G, lay.k)
    assert [len({r for r, _ in w.chunks}) for w in waves if w.op == "store"] == [75, 75, 75, 31]
