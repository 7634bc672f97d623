"""The decode page schedule (dsa_logits_schedule, and the one the forward
pass builds inside its quantisation launch): logits scored with it equal
dsa_indexer_logits bit for bit -- the schedule only decides which wave
scores which page -- for every knob value that changes its layout, for
batches of one and two 64-row position chunks, rows sharing requests, an
out-of-range position, and one schedule reused by two layers' inputs."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _reset():
    binding.dsa_device_error_flags(reset=True)
    yield
    for key in ("logits_kernel", "row_pages_per_wave", "row_head_waves"):
        binding.dsa_set_option(key, 0)


def _multi_row():
    rng = np.random.Generator(np.random.PCG64(515))
    ctx = rng.integers(100, 3000, 30).tolist()
    pos = [[L - 1] if r % 3 else [L - 2, L - 1] for r, L in enumerate(ctx)]
    return synth.build_batch(rng, ctx, pos, H=32, k=512)


BATCHES = {
    "decode64": lambda: synth.decode(),
    "decode100": lambda: synth.decode(R=100, seed=8),
    "decode128": lambda: synth.decode(R=128, seed=9),
    "short": lambda: synth.decode(R=40, lo=1, hi=300, seed=10),
    "multi_row": _multi_row,
}


def _scheduled(b, d, q8, qs, lg_out=None):
    sch = binding.dsa_logits_schedule(d["block_table"], d["qsl"],
                                      d["positions"], b.ld)
    assert sch is not None
    return binding.dsa_indexer_logits_scheduled(
        q8, qs, d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], b.ld, sch, logits=lg_out), sch


@pytest.mark.parametrize("name", sorted(BATCHES))
@pytest.mark.parametrize("ppw", [0, 2, 3, 4])
def test_scheduled_logits_equal_plain_logits(name, ppw):
    _say(f"case: scheduled logits, {name}, row_pages_per_wave {ppw}")
    binding.dsa_set_option("row_pages_per_wave", ppw)
    b = BATCHES[name]()
    d = parity.upload(b)
    q8, qs = binding.dsa_quantize_q(d["q_bf16"])
    plain = torch.full((b.T, b.ld), 7.0, device="cuda")
    binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                               d["block_table"], d["qsl"], d["positions"],
                               b.ld, plain)
    lg = torch.full((b.T, b.ld), 7.0, device="cuda")
    _scheduled(b, d, q8, qs, lg)
    torch.cuda.synchronize()
    assert torch.equal(lg, plain)          # values and untouched columns
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_schedule_reused_by_two_layers():
    """Two layers with their own q, weights and K cache over one batch's
    metadata: one schedule serves both."""
    _say("case: one schedule, two layers")
    layers = synth.index_cache_layers([0, 1], R=32, context=3000, H=64,
                                      k=256)
    b0, b1 = layers[0], layers[1]
    d0, d1 = parity.upload(b0), parity.upload(b1)
    sch = binding.dsa_logits_schedule(d0["block_table"], d0["qsl"],
                                      d0["positions"], b0.ld)
    for b, d in ((b0, d0), (b1, d1)):
        q8, qs = binding.dsa_quantize_q(d["q_bf16"])
        ref = torch.full((b.T, b.ld), 7.0, device="cuda")
        binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                                   d0["block_table"], d0["qsl"],
                                   d0["positions"], b.ld, ref)
        lg = torch.full((b.T, b.ld), 7.0, device="cuda")
        binding.dsa_indexer_logits_scheduled(
            q8, qs, d["weights"], d["k_cache"], d0["block_table"], d0["qsl"],
            d0["positions"], b.ld, sch, logits=lg)
        torch.cuda.synchronize()
        assert torch.equal(lg, ref)


def test_schedule_with_an_out_of_range_position():
    """A position past the logits row: the schedule builder flags it and
    gives it no pages; the other rows are as without a schedule."""
    _say("case: schedule, position past the row")
    b = synth.decode(R=16, seed=78)
    d = parity.upload(b)
    pos = d["positions"].clone()
    pos[3] = b.ld + 5
    d2 = dict(d, positions=pos)
    q8, qs = binding.dsa_quantize_q(d["q_bf16"])
    plain = torch.full((b.T, b.ld), 7.0, device="cuda")
    binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                               d["block_table"], d["qsl"], pos, b.ld, plain)
    assert binding.dsa_device_error_flags(reset=True) & 2
    lg = torch.full((b.T, b.ld), 7.0, device="cuda")
    _scheduled(b, d2, q8, qs, lg)
    torch.cuda.synchronize()
    assert binding.dsa_device_error_flags(reset=True) & 2
    assert torch.equal(lg, plain)
    assert torch.all(lg[3] == 7.0)


def test_no_schedule_for_wide_batches():
    """More than 128 rows: no schedule (size 0, nothing to build)."""
    assert binding.dsa_logits_schedule_size(129, 8192) == 0
    assert binding.dsa_logits_schedule_size(128, 8192) > 0


@pytest.mark.parametrize("name", ["decode64", "decode100", "multi_row"])
@pytest.mark.parametrize("ppw", [0, 2, 4])
def test_forward_with_its_schedule_equals_separate_calls(name, ppw):
    """The forward builds the schedule in its quantisation launch (D <= 3)
    or runs without it (D = 4): logits and top-k equal the three separate
    calls bit for bit."""
    _say(f"case: forward vs calls, {name}, row_pages_per_wave {ppw}")
    binding.dsa_set_option("row_pages_per_wave", ppw)
    b = BATCHES[name]()
    d = parity.upload(b)
    _, _, lg_ref, tk_ref = parity.run_gpu(b, d)
    lg, tk = binding.dsa_indexer_forward(d["q_bf16"], d["weights"],
                                         d["k_cache"], d["block_table"],
                                         d["qsl"], d["positions"], b.ld, b.k)
    torch.cuda.synchronize()
    assert torch.equal(tk, tk_ref)
    for t in range(b.T):
        p = int(b.positions[t])
        assert torch.equal(lg[t, : p + 1], lg_ref[t, : p + 1])
    assert binding.dsa_device_error_flags(reset=True) == 0
