"""GPU parity of the sparse-attention hand-off through the C ABI: top-k
rows as physical slots and as the 0 / -inf score mask, against the oracle,
exactly."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import handoff
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_handoff_on_decode_topk():
    """The decode batch's real top-k rows (some padded with -1)."""
    _say("case: hand-off on the decode batch's top-k")
    b = synth.decode(R=20, lo=1500, hi=4000, seed=3)
    d = parity.upload(b)
    _, _, _, tk = parity.run_gpu(b, d)
    slots = binding.dsa_topk_to_slots(tk, d["block_table"], d["qsl"])
    mask = binding.dsa_topk_mask(tk, b.ld)
    torch.cuda.synchronize()
    tkh = tk.cpu().numpy()
    assert np.array_equal(slots.cpu().numpy(),
                          handoff.topk_to_slots(tkh, b.block_table,
                                                b.query_start_loc))
    assert np.array_equal(mask.cpu().numpy(), handoff.topk_mask(tkh, b.ld))


@pytest.mark.parametrize("ld", [256, 16384, 16640, 40960])
def test_handoff_random_rows_and_chunk_edges(ld):
    """Random rows: indices on the 16384-column chunk edges, -1 padding,
    out-of-block-table indices, several requests per batch."""
    _say(f"case: hand-off, random rows, ld {ld}")
    rng = np.random.default_rng(ld)
    T, k, R = 40, 300 if ld > 256 else 64, 3
    pages = (ld + 63) // 64
    bt = rng.permutation(R * pages + 7).astype(np.int32)[:R * pages] \
        .reshape(R, pages)
    bt[1, pages // 2:] = -1
    qsl = np.array([0, 10, 25, T], dtype=np.int32)
    topk = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = rng.integers(0, k + 1)
        cols = rng.choice(ld, n, replace=False)
        edge = [c for c in (0, ld - 1, 16383, 16384) if c < ld]
        cols = np.unique(np.concatenate([cols, edge]))[:k]
        topk[t, :cols.size] = np.sort(cols)
    tk = torch.from_numpy(topk).cuda()
    slots = binding.dsa_topk_to_slots(tk, torch.from_numpy(bt).cuda(),
                                      torch.from_numpy(qsl).cuda())
    mask = binding.dsa_topk_mask(tk, ld)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(),
                          handoff.topk_to_slots(topk, bt, qsl))
    assert np.array_equal(mask.cpu().numpy(), handoff.topk_mask(topk, ld))


def test_handoff_uses_only_k_entries_of_a_wider_buffer():
    """topk_ld > k (the shared buffer wider than the rows' k): the entries
    past k hold decoy indices and must be ignored; slots keep row stride k."""
    _say("case: hand-off, k entries of a wider top-k buffer")
    rng = np.random.default_rng(77)
    T, k, extra, R, ld = 24, 100, 28, 2, 4096
    pages = ld // 64
    bt = rng.permutation(R * pages).astype(np.int32).reshape(R, pages)
    qsl = np.array([0, 9, T], dtype=np.int32)
    topk = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        n = int(rng.integers(0, k + 1))
        topk[t, :n] = np.sort(rng.choice(ld, n, replace=False))
    wide = np.concatenate(
        [topk, rng.integers(0, ld, (T, extra)).astype(np.int32)], axis=1)
    tk = torch.from_numpy(wide).cuda()
    slots = binding.dsa_topk_to_slots(tk, torch.from_numpy(bt).cuda(),
                                      torch.from_numpy(qsl).cuda(), k=k)
    mask = binding.dsa_topk_mask(tk, ld, k=k)
    torch.cuda.synchronize()
    assert slots.shape == (T, k)
    assert np.array_equal(slots.cpu().numpy(),
                          handoff.topk_to_slots(topk, bt, qsl))
    assert np.array_equal(mask.cpu().numpy(), handoff.topk_mask(topk, ld))
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_handoff_junk_indices():
    """Entries that name no cached token -- negative values other than -1,
    indices at or past ld and past the block table, INT32_MAX/MIN -- give
    slot -1 and no mask column, as in the oracle; valid entries beside them
    are unaffected."""
    _say("case: hand-off, junk indices")
    rng = np.random.default_rng(5)
    T, k, R, ld = 12, 64, 2, 16640
    pages = ld // 64
    bt = rng.permutation(R * pages).astype(np.int32).reshape(R, pages)
    qsl = np.array([0, 5, T], dtype=np.int32)
    junk = np.array([-7, -(2 ** 31), ld, ld + 100, 20000, 2 ** 31 - 1,
                     pages * 64, -2], dtype=np.int32)
    topk = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        good = np.sort(rng.choice(ld, 40, replace=False))
        row = np.concatenate([good, junk])
        rng.shuffle(row)
        topk[t, :row.size] = row
    tk = torch.from_numpy(topk).cuda()
    slots = binding.dsa_topk_to_slots(tk, torch.from_numpy(bt).cuda(),
                                      torch.from_numpy(qsl).cuda())
    mask = binding.dsa_topk_mask(tk, ld)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(),
                          handoff.topk_to_slots(topk, bt, qsl))
    assert np.array_equal(mask.cpu().numpy(), handoff.topk_mask(topk, ld))
    assert binding.dsa_device_error_flags(reset=True) == 0
