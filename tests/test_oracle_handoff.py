"""Pins for the oracle's sparse-attention hand-off (CPU only)."""

import json
import os

import numpy as np

from oracle import handoff, k_write

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slots_of_the_printed_block_row():
    """Logical positions as top-k entries map to the hand-computed slots of
    the printed block row [3, 7, 12] (the write path's golden fixture)."""
    g = json.load(open(os.path.join(GOLDEN, "slot_mapping_example.json")))
    bt = np.array([g["block_row"] + [-1]], dtype=np.int32)
    topk = np.array([g["positions"] + [-1]], dtype=np.int32)
    qsl = np.array([0, 1], dtype=np.int32)
    assert list(handoff.topk_to_slots(topk, bt, qsl)[0]) == g["slots"] + [-1]


def test_slots_are_where_the_write_path_stored_the_tokens():
    """For every selected index, the slot equals the slot the write path
    computes for that token of the same request."""
    rng = np.random.default_rng(5)
    bt = rng.permutation(64).astype(np.int32)[:40].reshape(4, 10)
    qsl = np.array([0, 2, 3, 3, 6], dtype=np.int32)
    topk = rng.integers(-1, 640, size=(6, 50)).astype(np.int32)
    slots = handoff.topk_to_slots(topk, bt, qsl)
    req = [0, 0, 1, 3, 3, 3]
    for t in range(6):
        for j in range(50):
            idx = int(topk[t, j])
            if idx < 0:
                assert slots[t, j] == -1
                continue
            # the write path: request req[t], position idx
            one = k_write.slot_mapping(bt[req[t]:req[t] + 1],
                                       np.array([0, 1], np.int32),
                                       np.array([idx], np.int32))
            assert slots[t, j] == one[0]


def test_mask_softmax_keeps_exactly_the_selected_set():
    rng = np.random.default_rng(8)
    T, ld, k = 5, 512, 37
    topk = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = [k, k, 10, 0, k][t]
        topk[t, :n] = np.sort(rng.choice(ld, n, replace=False))
    mask = handoff.topk_mask(topk, ld)
    score = rng.standard_normal((T, ld))
    for t in range(T):
        sel = topk[t][topk[t] >= 0]
        assert np.count_nonzero(mask[t] == 0) == sel.size
        assert np.all(np.isneginf(np.delete(mask[t], sel)))
        if sel.size == 0:
            continue
        z = score[t] + mask[t]
        p = np.exp(z - z[sel].max())
        p /= p.sum()
        q = np.exp(score[t][sel] - score[t][sel].max())
        q /= q.sum()
        assert np.all(p[np.setdiff1d(np.arange(ld), sel)] == 0)
        assert np.allclose(p[sel], q, rtol=1e-12, atol=0)
