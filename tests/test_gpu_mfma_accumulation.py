"""How exactly the FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) sums its 128
products, measured through the logits entry point on inputs where every
other step is exact.

With one head, weight 2, a q block whose largest element is 448 (so its
scale is exactly 1 and its codes are its values) and K scales of 1, the
logit of token s is 2 * max(d_s, 0) with d_s the MFMA's fp32 output for the
dot product of the q codes with the key codes: the weight folding (w * s_q /
2 = 1), the ReLU, the head sum (the other heads have weight 0) and the K
scale are all exact.  The exact dot is a multiple of 2^-18 (e4m3 values are
multiples of 2^-9), summed exactly in float64 here.

Measured on gfx950 (and pinned below): the MFMA does not return the
correctly rounded fp32 sum -- most dots differ from it -- and its error
grows with the spread of the products' magnitudes.  On codes drawn like the
workloads' (absmax-scaled normal values) it stays below 2^-16 of the sum of
the products' magnitudes, the absolute term of the parity tests' logits
tolerance; on codes spread over the whole e4m3 range it reaches about
2^-12.4 of it.  A plain fp32 sum of the same products (any order) would be
within about 2^-24 * 128 of that sum."""

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


def _codes_like_workload(rng, shape):
    """e4m3 codes of N(0,1) vectors scaled by their absmax to 448 (the
    workloads' quantisation; torch's cast rounds to nearest even)."""
    x = rng.standard_normal(shape).astype(np.float32)
    s = np.max(np.abs(x), axis=-1, keepdims=True) / np.float32(448.0)
    y = np.clip(x / s, -448, 448).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8) \
        .numpy()


def _case(seed, R, n, kind):
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "workload":
        q_codes = _codes_like_workload(rng, (R, 128))
        k_codes = _codes_like_workload(rng, (R, n, 128))
    else:
        q_codes = rng.choice(FINITE, size=(R, 128))
        k_codes = rng.choice(FINITE, size=(R, n, 128))
    q_codes[:, 0] = 0x7E                # largest q element 448: scale 1
    if kind == "cancel":
        # halves of q equal, second half of each key the negated first
        # half with 5 % of the codes nudged by one step: dots small
        # against their magnitudes
        q_codes[:, 64:] = q_codes[:, :64]
        k_codes[:, :, 64:] = k_codes[:, :, :64] ^ 0x80
        k_codes[:, :, 64:] ^= (rng.random((R, n, 64)) < 0.05).astype(
            np.uint8) * 0x01
        k_codes[(k_codes & 0x7F) == 0x7F] ^= 0x02  # NaN code -> 0x7D / 0xFD
    qv = DEC[q_codes]
    kv = DEC[k_codes]
    pages_per = (n + 63) // 64
    pool = R * pages_per
    bt = rng.permutation(pool).astype(np.int32).reshape(R, pages_per)
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


# kind -> the bound on |d - exact| / sum|products| that the hardware keeps
BOUNDS = {"workload": 2.0 ** -16, "full_range": 2.0 ** -11,
          "cancel": 2.0 ** -11}


@pytest.mark.parametrize("kind", sorted(BOUNDS))
def test_fp8_mfma_dot_error(kind):
    R, n = 16, 4096
    print(f"case: MFMA accumulation, {R} rows x {n} keys, {kind} codes",
          flush=True)
    sys.stdout.flush()
    q, kc, bt, exact, mag = _case(123 + sorted(BOUNDS).index(kind), R, n,
                                  kind)
    dev = "cuda"
    q8, qs = binding.dsa_quantize_q(q.to(dev))
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
    # compare where the MFMA's ReLU input is known to be positive: the
    # exact dot above the error bound (below it the clamp may go either way)
    bound = BOUNDS[kind]
    sure = exact > bound * mag
    err = np.abs(g[sure] - exact[sure])
    rel = err / mag[sure]
    rn32 = exact[sure].astype(np.float32).astype(np.float64)
    not_rn = float(np.mean(g[sure] != rn32))
    qq = np.quantile(rel, [0.5, 0.99, 1.0])
    print(f"{kind}: error / sum|products| median 2^{math.log2(qq[0] + 1e-300):.1f}, "
          f"p99 2^{math.log2(qq[1] + 1e-300):.1f}, max 2^{math.log2(qq[2] + 1e-300):.1f}; "
          f"{100 * not_rn:.1f} % of {int(sure.sum())} dots differ from the "
          "correctly rounded fp32 sum", flush=True)
    assert np.all(err <= bound * mag[sure])
    # a dot clearly below zero is clamped to exactly 0 by the ReLU
    assert np.all(g[exact < -bound * mag] == 0.0)


def test_fp8_mfma_rate_probe_counts_and_runs():
    """The measurement helper: its FLOP count is two 4-wave workgroups per
    compute unit x iters x 8 MFMAs x 2*16*16*128, and the launch it enqueues
    runs (a positive rate no higher than the chip's unit count allows)."""
    print("case: fp8 mfma rate probe", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    binding.dsa_fp8_mfma_rate_probe(iters)               # warm
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record()
    flops = binding.dsa_fp8_mfma_rate_probe(iters)
    z.record()
    torch.cuda.synchronize()
    assert flops == 2 * cus * 4 * iters * 8 * 2 * 16 * 16 * 128
    rate = flops / (a.elapsed_time(z) * 1e-3)
    # at most one 16x16x128 FP8 MFMA per 16 cycles per SIMD at 3 GHz
    assert 0 < rate < cus * 4 * (2 * 16 * 16 * 128 / 16) * 3e9



def test_page_read_probe_runs_on_any_ids():
    """The bare-read measurement helper reads the pages it is given, and ids
    outside the pool (negative, past the end) read nothing: no fault, no
    flag, and the cache is left as it was."""
    print("case: page read probe", flush=True)
    num_pages = 300
    cache = torch.randint(0, 255, (num_pages, 8448), dtype=torch.uint8,
                          device="cuda")
    before = cache.clone()
    ids = torch.tensor(list(range(0, num_pages, 7)) +
                       [-1, num_pages, num_pages + 5, -(1 << 30),
                        (1 << 31) - 1, 0], dtype=torch.int32, device="cuda")
    for n in (1, 2, 3, 4, ids.numel()):
        binding.dsa_page_read_probe(cache, ids[:n])
    binding.dsa_page_read_probe(cache, ids[:0])
    torch.cuda.synchronize()
    assert torch.equal(cache, before)
    assert binding.dsa_device_error_flags(reset=True) == 0
