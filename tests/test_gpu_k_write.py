"""GPU parity of the indexer-K write path through the C ABI: slot mapping
and the quantise-and-scatter kernel against the oracle, byte for byte."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import k_write as ok

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_keys(rng, n, scale=1.0):
    k = torch.from_numpy((rng.standard_normal((n, 128)) * scale)
                         .astype(np.float32)).bfloat16()
    return k, k.float().numpy()


def test_slot_mapping_matches_oracle():
    _say("case: slot mapping, 3 requests with padding rows")
    rng = np.random.default_rng(4)
    bt = rng.permutation(40).astype(np.int32)[:30].reshape(3, 10)
    bt[2, 7:] = -1
    qsl = np.array([0, 5, 5, 300], dtype=np.int32)
    pos = np.concatenate([rng.integers(0, 640, 5), rng.integers(0, 700, 295)]) \
        .astype(np.int32)
    pos[[3, 100]] = -1
    ref = ok.slot_mapping(bt, qsl, pos)
    got = binding.dsa_slot_mapping(torch.from_numpy(bt).cuda(),
                                   torch.from_numpy(qsl).cuda(),
                                   torch.from_numpy(pos).cuda())
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000])
def test_k_write_bytes_match_oracle(n):
    """Random keys (one all-zero, one tiny, one huge) into distinct random
    slots of a pre-filled pool, some padding slots: every byte of the pool
    equals the oracle's."""
    _say(f"case: k write, {n} tokens")
    rng = np.random.default_rng(n)
    num_pages = 24
    k_t, k_f = _bf16_keys(rng, n, 3.0)
    if n > 3:
        k_t[0] = 0
        k_t[1] *= 1e-6
        k_t[2] *= 1e4
        k_f = k_t.float().numpy()
    slots = rng.permutation(num_pages * 64)[:n].astype(np.int64)
    slots[rng.random(n) < 0.1] = -1
    pool = rng.integers(0, 256, (num_pages, 8448), dtype=np.uint8)
    ref = ok.write_k_cache(pool.copy(), k_f, slots)
    cache = torch.from_numpy(pool).cuda()
    binding.dsa_indexer_k_write(k_t.cuda(), torch.from_numpy(slots).cuda(),
                                cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    assert np.array_equal(got, ref), \
        f"{np.count_nonzero(got != ref)} bytes differ"
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_k_write_then_logits_equal_a_synth_cache():
    """Keys written through the C ABI, addressed by dsa_slot_mapping, give
    the same logits as the same keys laid out by the oracle's write."""
    _say("case: k write -> logits, decode-shaped")
    b = synth.decode(R=6, lo=100, hi=700, k=64, seed=21, pool_pages=80)
    rng = np.random.default_rng(21)
    L = [int(p) + 1 for p in b.positions]
    k_t, k_f = _bf16_keys(rng, sum(L), 1.0)
    rows, poss = [], []
    for r, n in enumerate(L):
        rows += [r] * n
        poss += list(range(n))
    qsl = np.r_[0, np.cumsum(L)].astype(np.int32)
    pos_all = np.array(poss, dtype=np.int32)
    slots = binding.dsa_slot_mapping(torch.from_numpy(b.block_table).cuda(),
                                     torch.from_numpy(qsl).cuda(),
                                     torch.from_numpy(pos_all).cuda())
    assert np.array_equal(slots.cpu().numpy(),
                          ok.slot_mapping(b.block_table, qsl, pos_all))
    pool = np.zeros_like(b.k_cache)
    ref_pool = ok.write_k_cache(pool.copy(), k_f, slots.cpu().numpy())
    cache = torch.from_numpy(pool).cuda()
    binding.dsa_indexer_k_write(k_t.cuda(), slots, cache)
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy(), ref_pool)
    q8, qs = binding.dsa_quantize_q(b.q_bf16.cuda())
    args = (q8, qs, torch.from_numpy(b.weights).cuda())
    tail = (torch.from_numpy(b.block_table).cuda(),
            torch.from_numpy(b.query_start_loc).cuda(),
            torch.from_numpy(b.positions).cuda(), b.ld)
    lg_gpu_cache = binding.dsa_indexer_logits(*args, cache, *tail)
    lg_ref_cache = binding.dsa_indexer_logits(
        *args, torch.from_numpy(ref_pool).cuda(), *tail)
    torch.cuda.synchronize()
    for t in range(b.T):
        p = int(b.positions[t])
        assert torch.equal(lg_gpu_cache[t, : p + 1], lg_ref_cache[t, : p + 1])


def test_k_write_slot_past_pool_is_flagged():
    _say("case: k write with a slot past the pool (host-forced)")
    rng = np.random.default_rng(2)
    k_t, k_f = _bf16_keys(rng, 4)
    pool = np.zeros((2, 8448), np.uint8)
    slots = np.array([5, 2 * 64, 70, -1], dtype=np.int64)   # 128 is past
    cache = torch.from_numpy(pool.copy()).cuda()
    binding.dsa_device_error_flags(reset=True)
    binding.dsa_indexer_k_write(k_t.cuda(), torch.from_numpy(slots).cuda(),
                                cache)
    assert binding.dsa_device_error_flags(reset=True) & 1
    keep = slots.copy()
    keep[1] = -1
    ref = ok.write_k_cache(pool.copy(), k_f, keep)
    assert np.array_equal(cache.cpu().numpy(), ref)
