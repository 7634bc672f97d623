"""dsa_indexer_forward_noalloc (the forward pass with the library's own
fixed scratch array instead of a caller workspace) through the C ABI: equal
to dsa_indexer_forward bit for bit on consecutive calls whose scratch needs
shrink (a 131072-column batch that uses the long-row top-k scratch, then
the decode batch, then the tiny batch), and a batch beyond the scratch
limit rejected before anything is enqueued."""

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


def _long_rows():
    rng = np.random.Generator(np.random.PCG64(31))
    ctx = 131072
    return synth.build_batch(rng, [ctx], [[ctx - 3, ctx - 2, ctx - 1]], H=64,
                             k=2048, name="noalloc_long")


def _both(b):
    d = parity.upload(b)
    T, ld, k = b.T, b.ld, b.k
    lg_ref, tk_ref = binding.dsa_indexer_forward(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], ld, k)
    lg = torch.full((T, ld), 5.0, dtype=torch.float32, device="cuda")
    tk = torch.full((T, k), 9, dtype=torch.int32, device="cuda")
    binding.dsa_indexer_forward_noalloc(
        d["q_bf16"], d["weights"], d["k_cache"], d["block_table"], d["qsl"],
        d["positions"], lg, tk)
    torch.cuda.synchronize()
    return lg_ref, tk_ref, lg, tk


def test_noalloc_forward_equals_forward_on_shrinking_batches():
    binding.dsa_device_error_flags(reset=True)
    for name, make in (("131072-column rows", _long_rows),
                       ("decode batch", synth.decode),
                       ("tiny", synth.tiny)):
        b = make()
        need = binding.dsa_forward_workspace_size(b.T, b.H, b.ld, b.k)
        _say(f"case: noalloc forward, {name} (T={b.T}, ld={b.ld}, scratch "
             f"{need} B)")
        assert need <= binding.NOALLOC_SCRATCH_BYTES
        lg_ref, tk_ref, lg, tk = _both(b)
        assert torch.equal(tk, tk_ref), name
        for t in range(b.T):
            p = int(b.positions[t])
            assert torch.equal(lg[t, : p + 1], lg_ref[t, : p + 1]), name
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_noalloc_forward_rejects_a_batch_beyond_its_scratch():
    _say("case: noalloc forward, 8192 rows x 64 heads (64 MiB of q codes)")
    T, H, ld, k = 8192, 64, 256, 32
    assert binding.dsa_forward_workspace_size(T, H, ld, k) > \
        binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    kc = torch.zeros((4, 8448), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    qsl = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    pos = torch.zeros((T,), dtype=torch.int32, device="cuda")
    lg = torch.full((T, ld), 5.0, dtype=torch.float32, device="cuda")
    tk = torch.full((T, k), 9, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.DsaError) as e:
        binding.dsa_indexer_forward_noalloc(q, w, kc, bt, qsl, pos, lg, tk)
    assert e.value.status == binding.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(lg == 5.0) and torch.all(tk == 9)
