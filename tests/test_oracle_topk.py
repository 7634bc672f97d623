"""Pins for the oracle's top-k and shared-buffer write (CPU only)."""

import numpy as np
import pytest

from oracle import indexer


def _argmax_rounds(v, k):
    """k rounds of argmax (first occurrence), removing the winner each time."""
    v = np.array(v, dtype=np.float64)
    out = []
    for _ in range(min(k, v.size)):
        i = int(np.argmax(v))
        out.append(i)
        v[i] = -np.inf
    return out


@pytest.mark.parametrize("n,k", [(1, 1), (5, 1), (50, 7), (300, 32),
                                 (64, 64), (65, 64), (1000, 999)])
def test_topk_vs_argmax_rounds(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    v = rng.standard_normal(n)
    got = indexer.topk_row(v, k)
    if n <= k:
        assert list(got[:n]) == list(range(n))
        assert np.all(got[n:] == -1)
    else:
        assert list(got) == _argmax_rounds(v, k)


def test_topk_with_ties_and_zeros():
    rng = np.random.default_rng(3)
    v = rng.integers(-3, 4, size=400).astype(np.float64)    # many exact ties
    v[v == 0] = np.where(rng.random((v == 0).sum()) < 0.5, 0.0, -0.0)
    for k in [1, 10, 57, 200, 399]:
        assert list(indexer.topk_row(v, k)) == _argmax_rounds(v, k)


def test_topk_k1_is_argmax():
    rng = np.random.default_rng(4)
    for _ in range(20):
        v = rng.standard_normal(777)
        assert indexer.topk_row(v, 1)[0] == np.argmax(v)


def test_topk_all_equal_takes_lowest_indices():
    v = np.full(100, 2.5)
    assert list(indexer.topk_row(v, 10)) == list(range(10))


def test_topk_padding_when_context_below_k():
    for n, k in [(1, 2048), (1023, 2048), (2047, 2048), (2048, 2048)]:
        got = indexer.topk_row(np.random.default_rng(n).standard_normal(n), k)
        assert got.shape == (k,) and got.dtype == np.int32
        assert sorted(got[:n].tolist()) == list(range(n))
        assert np.all(got[n:] == -1)


def test_topk_set_vs_argpartition():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(50000)
    k = 2048
    ref = np.argpartition(-v, k - 1)[:k]
    assert set(indexer.topk_row(v, k).tolist()) == set(ref.tolist())


def test_indexer_topk_reads_only_visible_columns():
    rng = np.random.default_rng(10)
    lg = rng.standard_normal((3, 512))
    lg[:, 100:] = 1e9            # garbage past p must be ignored
    pos = np.array([99, 50, 10], np.int32)
    out = indexer.indexer_topk(lg, pos, 8)
    for t in range(3):
        assert np.all(out[t] <= pos[t])
        assert list(out[t]) == _argmax_rounds(lg[t, : pos[t] + 1], 8)


def test_write_buffer_clears_rows_to_minus_one():
    buf = np.full((6, 4), 77, np.int32)
    rows = np.array([[3, 1, -1, -1], [0, 2, 5, 4]], np.int32)
    indexer.write_buffer(buf, rows)
    assert np.array_equal(buf[:2], rows)
    assert np.all(buf[2:] == 77)         # rows beyond T untouched
    buf2 = np.full((2, 6), 77, np.int32)
    indexer.write_buffer(buf2, rows)
    assert np.all(buf2[:, 4:] == -1)     # row tail cleared to -1
