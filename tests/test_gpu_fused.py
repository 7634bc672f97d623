"""GPU tests of the fused forward (dsa_indexer_forward_fused, through the C
ABI): scoring with candidate filtering and the top-k of the candidates,
without a logits buffer.  Its top-k must equal dsa_indexer_forward's bit
for bit (same logits arithmetic, exact selection with ties lowest position
first) on the candidate path, on the rescue path (forced for every row, or
reached through slot overflow), for every sample stride, and on the
degenerate rows; sampled rows are also checked against the oracle."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]

FUSED_OPTIONS = ("fused_sample_stride", "fused_cand_cap",
                 "fused_force_rescue", "fused_select")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _default_options():
    for o in FUSED_OPTIONS + ("logits_kernel", "tile_pages_per_step"):
        binding.dsa_set_option(o, 0)
    binding.dsa_device_error_flags(reset=True)
    yield
    for o in FUSED_OPTIONS:
        binding.dsa_set_option(o, 0)


def _forward(d, b):
    _, ref = binding.dsa_indexer_forward(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], b.ld, b.k)
    torch.cuda.synchronize()
    return ref


def _fused(d, b, **opts):
    for key, v in opts.items():
        binding.dsa_set_option(key, v)
    try:
        out = torch.full((b.T, b.k), 99, dtype=torch.int32, device="cuda")
        binding.dsa_indexer_forward_fused(
            d["q_bf16"], d["weights"], d["k_cache"], d["block_table"],
            d["qsl"], d["positions"], b.ld, b.k, out=out)
        torch.cuda.synchronize()
    finally:
        for key in opts:
            binding.dsa_set_option(key, 0)
    return out


def _ragged(seed=77, k=512):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = [5000, 700, 3000, 64, 2200]
    nq = [300, 37, 1, 64, 171]
    pos = [sorted(rng.choice(c, n, replace=False).tolist())
           for c, n in zip(ctx, nq)]
    return synth.build_batch(rng, ctx, pos, H=64, k=k)


VARIANTS = {
    "candidates": {},
    "forced_rescue": {"fused_force_rescue": 1},
    "slot_overflow": {"fused_cand_cap": 8},
    "stride16": {"fused_sample_stride": 16},
    "stride64": {"fused_sample_stride": 64},
    "select_wave64": {"fused_select": 1},
    "select_wave80": {"fused_select": 2},
    "select_block": {"fused_select": 3},
}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_ragged_prefill_equals_forward(variant):
    """Five requests with 1..300 query rows each (rows shorter and longer
    than k, tiles cut by request ends): bit-identical to the forward."""
    _say(f"case: fused ragged prefill, {variant}")
    b = _ragged()
    d = parity.upload(b)
    ref = _forward(d, b)
    out = _fused(d, b, **VARIANTS[variant])
    assert torch.equal(out, ref)
    assert binding.dsa_device_error_flags(reset=True) == 0
    if variant == "candidates":
        rows = [0, 150, 299, 300, 336, 337, 401, b.T - 1]
        ora = parity.oracle_logits(b, rows=rows)
        o = out.cpu().numpy()
        for i, t in enumerate(rows):
            p = int(b.positions[t])
            parity.check_topk_row(o[t], ora[i, : p + 1], b.k, f"row {t}")


@pytest.mark.parametrize("H,k", [(16, 64), (20, 96), (48, 300), (64, 1)])
def test_head_counts_and_k(H, k):
    """Every head-count instance of the tile and rescue kernels (full and
    padded M-tiles) and k from 1 up, with and without the rescue path."""
    _say(f"case: fused H={H} k={k}")
    rng = np.random.Generator(np.random.PCG64(1000 + H + k))
    ctx = [3000, 1500]
    pos = [list(range(2900, 3000)), list(range(0, 1500, 37))]
    b = synth.build_batch(rng, ctx, pos, H=H, k=k)
    d = parity.upload(b)
    ref = _forward(d, b)
    assert torch.equal(_fused(d, b), ref)
    assert torch.equal(_fused(d, b, fused_force_rescue=1), ref)
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_constant_and_tied_rows():
    """Rows whose head weights are all zero score 0 at every column (every
    logit ties: the sample threshold admits the whole row, the slots
    overflow, the rescue takes positions 0..k-1); rows with weights of one
    head only and integer-valued logits tie in groups."""
    _say("case: fused constant and tied rows")
    rng = np.random.Generator(np.random.PCG64(5))
    b = synth.build_batch(rng, [6000], [list(range(5900, 6000))], H=64,
                          k=256)
    w = b.weights.copy()
    w[::3] = 0.0
    w[1::3, 1:] = 0.0
    b2 = synth.IndexerBatch(q_bf16=b.q_bf16, weights=w, k_cache=b.k_cache,
                            block_table=b.block_table,
                            query_start_loc=b.query_start_loc,
                            positions=b.positions, k=b.k, ld=b.ld)
    d = parity.upload(b2)
    ref = _forward(d, b2)
    out = _fused(d, b2)
    assert torch.equal(out, ref)
    o = out.cpu().numpy()
    assert np.array_equal(o[0], np.arange(256))


def test_out_of_range_rows_and_pages():
    """A row whose position is past its block-table row (a row of -1), a
    block-table entry outside the page pool (that page scores -inf; flagged
    by both calls), rows of at most k columns (0..p then -1)."""
    _say("case: fused out-of-range rows and pages")
    rng = np.random.Generator(np.random.PCG64(9))
    ctx = [4000, 300]
    pos = [list(range(3950, 4000)), list(range(200, 300, 3))]
    b = synth.build_batch(rng, ctx, pos, H=32, k=512)
    bt = b.block_table.copy()
    bt[0, 20] = b.k_cache.shape[0] + 5                 # outside the pool
    positions = b.positions.copy()
    positions[3] = bt.shape[1] * 64 + 10               # past the table row
    b2 = synth.IndexerBatch(q_bf16=b.q_bf16, weights=b.weights,
                            k_cache=b.k_cache, block_table=bt,
                            query_start_loc=b.query_start_loc,
                            positions=positions, k=b.k,
                            ld=max(b.ld, synth.round_up(int(positions[3]) + 1,
                                                        256)))
    d = parity.upload(b2)
    ref = _forward(d, b2)
    f_ref = binding.dsa_device_error_flags(reset=True)
    out = _fused(d, b2)
    f_out = binding.dsa_device_error_flags(reset=True)
    assert torch.equal(out, ref)
    assert f_ref == f_out and f_out != 0
    assert np.all(out.cpu().numpy()[3] == -1)


def test_non_tiled_batch_runs_the_forward():
    """T <= 2 R (a decode batch): the fused entry runs the forward with the
    logits in its workspace -- same rows."""
    _say("case: fused entry on a decode batch")
    b = synth.decode(R=16)
    d = parity.upload(b)
    assert torch.equal(_fused(d, b), _forward(d, b))


def test_workspace_is_smaller_than_the_logits_it_replaces():
    b_T, ld, k, H = 8192, 40960, 2048, 64
    fused = binding.dsa_forward_fused_workspace_size(b_T, 1, H, ld, k)
    plain = (binding.dsa_forward_workspace_size(b_T, H, ld, k) +
             b_T * ld * 4)
    assert 0 < fused < plain


def test_full_size_prefill():
    """The 8192 x 40960 prefill chunk: candidate path (every select kernel,
    sample strides 16 and 64) and forced rescue all bit-identical to the
    forward; 16 evenly spaced rows against the oracle."""
    _say("case: fused full-size prefill")
    b = synth.prefill()
    d = parity.upload(b)
    ref = _forward(d, b)
    out = _fused(d, b)
    assert torch.equal(out, ref)
    for sel in (1, 2, 3):
        _say(f"case: fused full-size prefill, select kernel {sel}")
        assert torch.equal(_fused(d, b, fused_select=sel), ref)
    for ss in (16, 64):
        _say(f"case: fused full-size prefill, sample stride {ss}")
        assert torch.equal(_fused(d, b, fused_sample_stride=ss), ref)
    _say("case: fused full-size prefill, forced rescue")
    assert torch.equal(_fused(d, b, fused_force_rescue=1), ref)
    assert binding.dsa_device_error_flags(reset=True) == 0
    rows = np.linspace(0, b.T - 1, 16).astype(np.int64)
    ora = parity.oracle_logits(b, rows=rows)
    o = out.cpu().numpy()
    for i, t in enumerate(rows):
        p = int(b.positions[t])
        parity.check_topk_row(o[t], ora[i, : p + 1], b.k, f"row {t}")


def test_full_size_long_context():
    """The 1M-token tail: 16 rows of 1,048,576 columns, candidate path and
    forced rescue bit-identical to the forward."""
    _say("case: fused 1M-token tail")
    b = synth.long_context()
    d = parity.upload(b)
    ref = _forward(d, b)
    assert torch.equal(_fused(d, b), ref)
    _say("case: fused 1M-token tail, forced rescue")
    assert torch.equal(_fused(d, b, fused_force_rescue=1), ref)
    assert binding.dsa_device_error_flags(reset=True) == 0
