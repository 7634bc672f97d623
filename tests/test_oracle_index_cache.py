"""Pins for the oracle's IndexCache F/S rule and layer loop (CPU only),
against the IndexCache guide's worked examples (tests/golden/)."""

import numpy as np
import pytest

from oracle import index_cache, indexer
from dsa_lightning_indexer_amd import synth


def _full(mask):
    return [i for i, s in enumerate(mask) if not s]


def test_freq4_offset2_61_layers(golden):
    g = golden("index_cache_examples.json")["freq4_offset2_61"]
    m = index_cache.skip_mask(g["num_layers"], freq=g["freq"], offset=g["offset"])
    assert _full(m) == g["full_layers"]
    assert len(_full(m)) == 16 and m.sum() == 45
    assert not m[0] and not m[1]


def test_printed_pattern(golden):
    g = golden("index_cache_examples.json")["pattern_61"]
    assert len(g["pattern"]) == g["length"]
    m = index_cache.skip_mask(61, pattern=g["pattern"], freq=4, offset=2)
    assert _full(m) == g["full_layers"]
    assert len(_full(m)) == g["num_full"]


def test_defaults_every_layer_full(golden):
    d = golden("index_cache_examples.json")["defaults"]
    m = index_cache.skip_mask(61, pattern=d["pattern"], freq=d["freq"],
                              offset=d["offset"])
    assert not m.any()


def test_pattern_overrides_freq_and_falls_back_past_its_length():
    m = index_cache.skip_mask(8, pattern="FSS", freq=2, offset=0)
    assert m.tolist() == [False, True, True] + [False] * 5


def test_mtp_layers_always_full():
    m = index_cache.skip_mask(64, pattern="F" + "S" * 63, num_hidden_layers=61)
    assert m[1:61].all() and not m[61:].any()
    m = index_cache.skip_mask(64, freq=4, offset=2, num_hidden_layers=61)
    assert not m[61:].any()
    assert m[60]                               # 59 % 4 != 0 -> S


def test_offset_zero_makes_layer0_skip_with_freq_gt1():
    # max(0 - 0 + 1, 0) % 2 = 1 -> S: the rule itself allows it ...
    assert index_cache.is_skip(0, freq=2, offset=0)
    # ... but a run must refuse it (it would read a never-written buffer)
    with pytest.raises(ValueError):
        index_cache.run([None, None], None, None, [0], 256, 4,
                        np.zeros((1, 4), np.int32), freq=2, offset=0)


@pytest.mark.parametrize("bad", [dict(freq=0), dict(pattern="FFX"),
                                 dict(pattern="fs")])
def test_invalid_configs_raise(bad):
    with pytest.raises(ValueError):
        index_cache.skip_mask(4, **bad)


def test_run_s_layers_reuse_previous_full_layer():
    rng = np.random.Generator(np.random.PCG64(21))
    base = synth.build_batch(rng, [200, 90], [[199], [70, 89]], H=4, k=16)
    layers = []
    for l in range(7):
        r = np.random.Generator(np.random.PCG64(100 + l))
        b = synth.build_batch(r, [200, 90], [[199], [70, 89]], H=4, k=16,
                              layout=(base.block_table, base.k_cache.shape[0]))
        layers.append({"q": b.q_f32, "weights": b.weights,
                       "k_cache": b.k_cache})
    buf0 = np.full((5, 16), 123, np.int32)
    mask, B, snaps = index_cache.run(
        layers, base.block_table, base.query_start_loc, base.positions,
        base.ld, 16, buf0, freq=3, offset=1)
    assert mask.tolist() == [False, True, True, False, True, True, False]
    assert np.array_equal(buf0, np.full((5, 16), 123))      # input untouched
    assert np.all(B[3:] == 123)                  # rows beyond T untouched
    last_full = None
    for l, s in enumerate(mask):
        if not s:
            lay = layers[l]
            codes, sc = indexer.quantize_q(lay["q"])
            lg = indexer.indexer_logits(codes, sc, lay["weights"],
                                        lay["k_cache"], base.block_table,
                                        base.query_start_loc, base.positions,
                                        base.ld)
            want = indexer.indexer_topk(lg, base.positions, 16)
            assert np.array_equal(snaps[l], want)
            last_full = l
        else:
            assert np.array_equal(snaps[l], snaps[last_full])
    # distinct layers really give distinct selections
    assert not np.array_equal(snaps[0], snaps[3])
