"""GPU tests of the row-chunked forward under a logits budget
(dsa_indexer_forward_chunked, through the C ABI): its top-k equals the
unchunked forward's bit for bit for every chunk size, in every logits
kernel class, with chunks that cut through requests; sampled rows against
the oracle."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import chunking
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(b, rows_list, budget=None):
    d = parity.upload(b)
    _, ref = binding.dsa_indexer_forward(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], b.ld, b.k)
    torch.cuda.synchronize()
    ref = ref.cpu().numpy()
    outs = {}
    for rows in rows_list:
        out = torch.full((b.T, b.k), 99, dtype=torch.int32, device="cuda")
        binding.dsa_indexer_forward_chunked(
            d["q_bf16"], d["weights"], d["k_cache"], d["block_table"],
            d["qsl"], d["positions"], b.ld, b.k, rows_per_chunk=rows,
            budget_bytes=budget, out=out)
        torch.cuda.synchronize()
        outs[rows] = out.cpu().numpy()
    assert binding.dsa_device_error_flags(reset=True) == 0
    return ref, outs


@pytest.mark.parametrize("rows", [1, 7, 64])
def test_decode_batch_chunked_equals_forward(rows):
    _say(f"case: chunked decode batch (balanced class), {rows} rows/chunk")
    b = synth.decode()
    ref, outs = _both(b, [rows])
    assert np.array_equal(outs[rows], ref)


def test_rowwise_class_chunked_equals_forward():
    """200 single-row requests: the whole batch takes the row-wise class;
    chunks of 64 and 13 rows keep it."""
    _say("case: chunked 200-row decode (row-wise class)")
    b = synth.decode(R=200, lo=300, hi=3000, k=256, seed=31)
    ref, outs = _both(b, [64, 13])
    for rows, o in outs.items():
        assert np.array_equal(o, ref), rows


def test_ragged_prefill_chunks_cut_requests():
    """Five requests with 1..300 query rows each (tiled class); chunk sizes
    that start and end inside requests and inside 16-row tiles."""
    _say("case: chunked ragged prefill (tiled class)")
    rng = np.random.Generator(np.random.PCG64(77))
    ctx = [5000, 700, 3000, 64, 2200]
    nq = [300, 37, 1, 64, 171]
    pos = [sorted(rng.choice(c, n, replace=False).tolist())
           for c, n in zip(ctx, nq)]
    b = synth.build_batch(rng, ctx, pos, H=64, k=512)
    ref, outs = _both(b, [1, 15, 16, 100, 333, b.T])
    for rows, o in outs.items():
        assert np.array_equal(o, ref), rows
    rows = [0, 299, 300, 336, 337, 401, b.T - 1]
    ora = parity.oracle_logits(b, rows=rows)
    for i, t in enumerate(rows):
        p = int(b.positions[t])
        parity.check_topk_row(outs[100][t], ora[i, : p + 1], b.k, f"row {t}")


def test_full_size_prefill_under_a_budget():
    """The 8192 x 40960 prefill chunk with a 256 MiB logits budget: the
    budget rule gives 1638 rows per chunk (6 chunks) -- equal to the
    unchunked forward bit for bit."""
    b = synth.prefill()
    budget = 256 << 20
    rows = binding.dsa_logits_chunk_rows(b.T, b.ld, budget)
    assert rows == chunking.chunk_rows(b.T, b.ld, budget) == 1638
    _say(f"case: full-size prefill, budget 256 MiB -> {rows} rows per chunk")
    d = parity.upload(b)
    _, ref = binding.dsa_indexer_forward(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], b.ld, b.k)
    out = binding.dsa_indexer_forward_chunked(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], b.ld, b.k, budget_bytes=budget)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert binding.dsa_device_error_flags(reset=True) == 0
