"""Seeded random small configurations through the C ABI against the oracle:
request counts, context lengths, query rows per request (one per request,
a few, many, or over a hundred single-row requests -- the balanced, tiled
and row-wise logits kernels), head
counts 1..64, index_topk from 1 to beyond the context, and row strides with
unused columns.  Every case: logits under the stated tolerance, top-k
within the tie window and exactly the top-k of the GPU's own logits."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]

HEADS = [1, 3, 4, 16, 20, 32, 48, 64]


def _case(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    # 0: 1 row/request, 1: a few, 2: many (tiled), 3: > 128 single-row
    # requests (row-wise logits)
    mode = seed % 4
    R = (int(rng.integers(129, 201)) if mode == 3 else
         int(rng.integers(1, 7 if mode < 2 else 5)))
    ctx, pos = [], []
    for _ in range(R):
        L = int(rng.integers(1, 600 if mode == 3 else 3000))
        ctx.append(L)
        if mode in (0, 3):
            pos.append([L - 1])
        else:
            m = int(rng.integers(1, 4 if mode == 1 else 41))
            m = min(m, L)
            pos.append(sorted(rng.choice(L, m, replace=False).tolist()))
    H = HEADS[seed % len(HEADS)]
    k = int(rng.choice([1, 7, 64, 300, 2048]))
    b = synth.build_batch(rng, ctx, pos, H=H, k=k,
                          boost_frac=0.02 if seed % 2 else 0.0)
    if seed % 4 == 3:                     # spare columns past every row
        b.ld += 256
    return b


@pytest.mark.parametrize("seed", range(120))
def test_random_configuration(seed):
    b = _case(seed)
    print(f"case: seed {seed}: R={b.R} T={b.T} H={b.H} k={b.k} ld={b.ld}",
          flush=True)
    sys.stdout.flush()
    binding.dsa_device_error_flags(reset=True)
    _, _, lg, tk = parity.run_gpu(b)
    lg, tk = lg.cpu().numpy(), tk.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_logits_row(lg[t], ora[t], p, f"seed {seed} row {t}",
                                mag[t])
        parity.check_topk_row(tk[t], ora[t, : p + 1], b.k,
                              f"seed {seed} row {t}")
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t], p, b.k,
                                              f"seed {seed} row {t}")
    assert binding.dsa_device_error_flags(reset=True) == 0
