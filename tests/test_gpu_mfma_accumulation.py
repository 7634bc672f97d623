"""How exactly the FP8 MFMA sums its 128 products, measured through the
logits entry point on inputs where every other step is exact.

With one head, weight 2, a q block whose largest element is 448 (so its
scale is exactly 1 and its codes are its values) and K scales of 1, the
logit of token s is 2 * max(d_s, 0) with d_s the MFMA's fp32 output for the
dot product of the q codes with the key codes: the weight folding (w * s_q /
2 = 1), the ReLU, the head sum (the other heads have weight 0) and the K
scale are all exact.  The exact dot is an integer multiple of 2^-18 (e4m3
values are multiples of 2^-9), summed exactly in float64 here.

The logits tolerance of the parity tests assumes the error of one such dot
stays below 2^-16 of the sum of the magnitudes of its products; this test
measures the error on random and on cancelling dot products and checks that
assumption, and prints how far the result is from a correctly rounded fp32
sum (plain fp32 accumulation would be within about 2^-24 relative of the
dot itself)."""

import math
import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import fp8

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]

DEC = fp8.decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
FINITE = np.array([c for c in range(256) if np.isfinite(DEC[c])], np.uint8)


def _case(seed, R, n, cancel):
    rng = np.random.Generator(np.random.PCG64(seed))
    # q: e4m3 values (exact in bf16), element 0 = 448 so the scale is 1
    q_codes = rng.choice(FINITE, size=(R, 128))
    q_codes[:, 0] = 0x7E
    if cancel:                        # halves equal: see the K codes below
        q_codes[:, 64:] = q_codes[:, :64]
    qv = DEC[q_codes]
    # K codes: random finite e4m3; "cancel" flips signs to pair products so
    # that the dots are small against their magnitudes
    k_codes = rng.choice(FINITE, size=(R, n, 128))
    if cancel:
        k_codes[:, :, 64:] = k_codes[:, :, :64] ^ 0x80
        k_codes[:, :, 64:] ^= (rng.random((R, n, 64)) < 0.05).astype(
            np.uint8) * 0x01                       # near, not exact, cancel
        k_codes[(k_codes & 0x7F) == 0x7F] ^= 0x02  # NaN code -> 0x7D / 0xFD
    kv = DEC[k_codes]
    pages_per = (n + 63) // 64
    pool = R * pages_per
    perm = rng.permutation(pool).astype(np.int32)
    bt = perm.reshape(R, pages_per)
    kc = np.zeros((pool, 8448), np.uint8)
    for r in range(R):
        codes = np.zeros((pages_per * 64, 128), np.uint8)
        codes[:n] = k_codes[r]
        kc[bt[r], :8192] = codes.reshape(pages_per, 8192)
        sc = np.zeros(pages_per * 64, np.float32)
        sc[:n] = 1.0
        kc[bt[r], 8192:] = sc.view(np.uint8).reshape(pages_per, 256)
    exact = np.einsum("ri,rni->rn", qv, kv)            # exact in float64
    mag = np.einsum("ri,rni->rn", np.abs(qv), np.abs(kv))
    q = torch.from_numpy(qv.astype(np.float32)).to(torch.bfloat16) \
        .reshape(R, 1, 128)
    return q, kc, bt, exact, mag


@pytest.mark.parametrize("cancel", [False, True])
def test_fp8_mfma_dot_error(cancel):
    R, n = 16, 4096
    print(f"case: MFMA accumulation, {R} rows x {n} keys, cancel={cancel}",
          flush=True)
    sys.stdout.flush()
    q, kc, bt, exact, mag = _case(123 + int(cancel), R, n, cancel)
    dev = "cuda"
    q = q.to(dev)
    q8, qs = binding.dsa_quantize_q(q)
    assert torch.all(qs == 1.0)
    w = torch.full((R, 1), 2.0, dtype=torch.float32, device=dev)
    qsl = torch.arange(R + 1, dtype=torch.int32, device=dev)
    pos = torch.full((R,), n - 1, dtype=torch.int32, device=dev)
    ld = synth.round_up(n, 256)
    lg = binding.dsa_indexer_logits(
        q8, qs, w, torch.from_numpy(kc).to(dev), torch.from_numpy(bt).to(dev),
        qsl, pos, ld)
    torch.cuda.synchronize()
    assert binding.dsa_device_error_flags(reset=True) == 0
    g = lg[:, :n].cpu().numpy().astype(np.float64) / 2.0
    pos_ = exact > 0
    err = np.abs(g[pos_] - exact[pos_])
    rel_m = err / mag[pos_]
    rn32 = exact[pos_].astype(np.float32).astype(np.float64)
    not_rn = float(np.mean(g[pos_] != rn32))
    rel_d = err / exact[pos_]
    q_m = np.quantile(rel_m, [0.5, 0.99, 1.0])
    print(f"MFMA dot error / sum|products|: median 2^{math.log2(q_m[0] + 1e-300):.1f}"
          f", p99 2^{math.log2(q_m[1] + 1e-300):.1f}, max 2^{math.log2(q_m[2] + 1e-300):.1f}; "
          f"relative to the dot: max {rel_d.max():.3g}; "
          f"{100 * not_rn:.1f} % of {pos_.sum()} positive dots differ from "
          f"the correctly rounded fp32 sum", flush=True)
    # negative dots are clamped to exactly 0
    assert np.all(g[~pos_ & (exact < 0)] == 0.0)
    # the premise of the parity tolerance
    assert np.all(err <= 2.0 ** -16 * mag[pos_])
