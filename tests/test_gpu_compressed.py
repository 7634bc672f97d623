"""GPU parity of the DeepSeek-V4 compressed-cache variant through the C ABI:
the compressed slot mapping against the oracle (exact), and a compressed
indexer cache written and scored end to end (keys at the compressed slots,
rows at their compressed positions) against the oracle."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding
from oracle import indexer as oi
from oracle import k_write as ok
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("ratio,bs", [(1, 64), (4, 64), (128, 2), (3, 5)])
def test_compressed_slot_mapping_matches_oracle(ratio, bs):
    _say(f"case: compressed slot mapping, ratio {ratio}, block {bs}")
    rng = np.random.default_rng(ratio * 100 + bs)
    bt = rng.permutation(60).astype(np.int32)[:36].reshape(3, 12)
    bt[1, 8:] = -1
    qsl = np.array([0, 400, 400, 1000], dtype=np.int32)
    span = 12 * bs * ratio + 3 * ratio               # some past the table
    pos = rng.integers(0, span, 1000).astype(np.int32)
    pos[:64] = np.arange(64) * ratio + ratio - 1     # boundary tokens
    pos[[5, 700]] = -1
    slots, pc = binding.dsa_compressed_slot_mapping(
        _dev(bt), _dev(qsl), _dev(pos), ratio, bs)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(),
                          ok.compressed_slot_mapping(bt, qsl, pos, ratio, bs))
    assert np.array_equal(pc.cpu().numpy(),
                          ok.compressed_positions(pos, ratio))


def test_compressed_slot_mapping_at_int32_extremes():
    """Positions up to 2^31 - 1: (p + 1) is formed in 64 bits."""
    _say("case: compressed slot mapping at int32 extremes")
    bt = np.arange(8, dtype=np.int32).reshape(1, 8)
    qsl = np.array([0, 6], dtype=np.int32)
    big = 2 ** 31 - 1
    pos = np.array([big, big - 1, big - 3, 3, 7, -1], dtype=np.int32)
    for ratio, bs in ((4, 64), (128, 2), (1, 64), (big, 1)):
        slots, pc = binding.dsa_compressed_slot_mapping(
            _dev(bt), _dev(qsl), _dev(pos), ratio, bs)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(),
                              ok.compressed_slot_mapping(bt, qsl, pos, ratio,
                                                         bs)), ratio
        assert np.array_equal(pc.cpu().numpy(),
                              ok.compressed_positions(pos, ratio)), ratio


def test_compressed_ratio_one_is_the_plain_kernel():
    _say("case: compressed slot mapping at ratio 1 vs dsa_slot_mapping")
    rng = np.random.default_rng(9)
    bt = rng.permutation(80).astype(np.int32)[:64].reshape(4, 16)
    qsl = np.array([0, 10, 300, 301, 2000], dtype=np.int32)
    pos = rng.integers(-1, 1100, 2000).astype(np.int32)
    a = binding.dsa_slot_mapping(_dev(bt), _dev(qsl), _dev(pos))
    b, _ = binding.dsa_compressed_slot_mapping(_dev(bt), _dev(qsl), _dev(pos),
                                               1, 64, want_positions_c=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_compressed_cache_written_and_scored():
    """Ratio 4, 256-token host blocks (64-entry storage blocks, the 8448-byte
    page): every token of three requests goes through the compressed slot
    mapping and dsa_indexer_k_write (only the boundary tokens store a key),
    then rows at their compressed positions are scored and ranked; cache
    bytes exactly, logits and top-k within the parity tolerances."""
    ratio, bs, H, k = 4, 64, 64, 128
    _say(f"case: compressed cache end to end, ratio {ratio}, H {H}, k {k}")
    rng = np.random.default_rng(44)
    ctx = [1203, 2600, 5000]                          # tokens per request
    n_c = [c // ratio for c in ctx]
    nblk = [-(-n // bs) for n in n_c]
    pool_pages = sum(nblk) + 7
    ids = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((3, max(nblk)), -1, np.int32)
    o = 0
    for r, n in enumerate(nblk):
        bt[r, :n] = ids[o:o + n]
        o += n
    qsl_k = np.r_[0, np.cumsum(ctx)].astype(np.int32)
    pos_k = np.concatenate([np.arange(c) for c in ctx]).astype(np.int32)
    keys = torch.from_numpy(rng.standard_normal((len(pos_k), 128))
                            .astype(np.float32)).bfloat16()
    slots, _ = binding.dsa_compressed_slot_mapping(
        _dev(bt), _dev(qsl_k), _dev(pos_k), ratio, bs,
        want_positions_c=False)
    ref_slots = ok.compressed_slot_mapping(bt, qsl_k, pos_k, ratio, bs)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert int((ref_slots >= 0).sum()) == sum(n_c)
    pool = rng.integers(0, 256, (pool_pages, 8448), dtype=np.uint8)
    ref_pool = ok.write_k_cache(pool.copy(), keys.float().numpy(), ref_slots)
    cache = _dev(pool)
    binding.dsa_indexer_k_write(keys.cuda(), slots, cache)
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy(), ref_pool)

    # query rows: the last token of each request and a few earlier ones
    qpos = [[c - 1, c - 2, ratio * 40 - 1, ratio * 300 + 1] for c in ctx]
    qsl_q = np.r_[0, np.cumsum([len(q) for q in qpos])].astype(np.int32)
    pos_q = np.array(sum(qpos, []), dtype=np.int32)
    _, pc = binding.dsa_compressed_slot_mapping(
        _dev(bt), _dev(qsl_q), _dev(pos_q), ratio, bs)
    pc_ref = ok.compressed_positions(pos_q, ratio).astype(np.int32)
    assert np.array_equal(pc.cpu().numpy(), pc_ref)
    T = len(pos_q)
    ld = -(-int(pc_ref.max() + 1) // 256) * 256
    q = torch.from_numpy(rng.standard_normal((T, H, 128)).astype(np.float32)
                         ).bfloat16()
    w = (rng.standard_normal((T, H)) / np.sqrt(H)).astype(np.float32)
    binding.dsa_device_error_flags(reset=True)
    q8, qs = binding.dsa_quantize_q(q.cuda())
    lg = binding.dsa_indexer_logits(q8, qs, _dev(w), cache, _dev(bt),
                                    _dev(qsl_q), pc, ld)
    tk = binding.dsa_indexer_topk(lg, pc, k)
    torch.cuda.synchronize()
    assert binding.dsa_device_error_flags(reset=True) == 0
    codes, s = oi.quantize_q(q.float().numpy())
    ref = oi.indexer_logits(codes, s, w, ref_pool, bt, qsl_q, pc_ref, ld)
    lg_h, tk_h = lg.cpu().numpy(), tk.cpu().numpy()
    req = oi.request_of_rows(qsl_q, T)
    for t in range(T):
        p = int(pc_ref[t])
        # the parity rule's summation term: M = sum_h |w| sum_i |qhat||khat|
        qa = np.abs(oi.dequantize(codes[t], s[t]))
        ka = np.abs(oi.gather_k(ref_pool, bt[req[t]], 0, p + 1))
        m = np.abs(w[t]).astype(np.float64) @ (qa @ ka.T)
        parity.check_logits_row(lg_h[t], ref[t], p, f"row {t}", m)
        parity.check_topk_row(tk_h[t], ref[t, : p + 1], k, f"row {t}")
        parity.check_topk_exact_on_gpu_logits(tk_h[t], lg_h[t], p, k,
                                              f"row {t}")
