"""Pins for the oracle's indexer-K write path (CPU only): slot mapping,
per-token FP8 quantisation and the scatter into 8448-byte pages."""

import json
import os

import numpy as np
import torch

from oracle import fp8, k_write
from oracle.indexer import PAGE_BYTES, PAGE_KEY_BYTES, HEAD_DIM, PAGE_TOKENS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slot_mapping_printed_block_row():
    """The printed block row [3, 7, 12] and the section 2.3 formula
    (golden fixture worked by hand)."""
    g = json.load(open(os.path.join(GOLDEN, "slot_mapping_example.json")))
    assert g["page_tokens"] == PAGE_TOKENS
    bt = np.array([g["block_row"] + [-1]], dtype=np.int32)   # padded row
    pos = np.array(g["positions"], dtype=np.int32)
    qsl = np.array([0, len(pos)], dtype=np.int32)
    assert list(k_write.slot_mapping(bt, qsl, pos)) == g["slots"]


def test_slot_mapping_two_requests_and_padding():
    bt = np.array([[5, -1], [2, 9]], dtype=np.int32)
    qsl = np.array([0, 2, 5], dtype=np.int32)
    pos = np.array([3, 64, 0, 70, -1], dtype=np.int32)
    # row 1 of request 0 is past its only block; row 4 has no position
    assert list(k_write.slot_mapping(bt, qsl, pos)) == \
        [5 * 64 + 3, -1, 2 * 64 + 0, 9 * 64 + 6, -1]


def test_write_offsets_by_hand():
    """Tokens of constant magnitude c: every code is 0x7E (|k|/s = 448),
    the scale is fp32(c / 448); their bytes land at page * 8448 + row * 128
    and page * 8448 + 8192 + row * 4, and nothing else changes."""
    num_pages = 3
    cache = np.full((num_pages, PAGE_BYTES), 0xA5, dtype=np.uint8)
    c = np.array([1.0, 2.0, 3.0, 4.0, 5.0], dtype=np.float32)
    k = np.repeat(c[:, None], HEAD_DIM, axis=1)
    k[1, ::2] *= -1                                  # signs: 0xFE codes
    slots = np.array([0, 63, 64, 130, -1], dtype=np.int64)
    k_write.write_k_cache(cache, k, slots)
    expect = np.full_like(cache, 0xA5)
    flat = expect.reshape(-1)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        page, row = slot // 64, slot % 64
        codes = np.where(k[i] < 0, 0xFE, 0x7E).astype(np.uint8)
        base = page * 8448
        flat[base + row * 128: base + row * 128 + 128] = codes
        sc = np.float32(c[i]) / np.float32(448.0)
        flat[base + 8192 + 4 * row: base + 8192 + 4 * row + 4] = \
            np.frombuffer(np.float32(sc).tobytes(), np.uint8)
    assert np.array_equal(cache, expect)


def test_quantize_error_bound_and_library_cast():
    """Round trip within half an e4m3 step (2^-4 relative in the normal
    range, 2^-10 * s below it); the codes equal torch's float32 ->
    float8_e4m3fn cast of fp32(k / s)."""
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((512, HEAD_DIM))
                         .astype(np.float32)).bfloat16().float().numpy()
    k[7] *= 1e-3
    codes, s = k_write.quantize_k(k)
    back = fp8.decode(codes) * s.astype(np.float64)[:, None]
    x = np.abs(k.astype(np.float64) / s.astype(np.float64)[:, None])
    bound = np.where(x >= 2.0 ** -6, x * 2.0 ** -4, 2.0 ** -10) * \
        s.astype(np.float64)[:, None]
    assert np.all(np.abs(back - k) <= bound * (1 + 1e-12))
    ref = torch.from_numpy((k / s[:, None]).astype(np.float32)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.all(np.max(codes & 0x7F, axis=1) == 0x7E)   # amax -> 448


def test_zero_key_stores_zero_scale():
    k = np.zeros((2, HEAD_DIM), np.float32)
    k[1, 5] = -0.5
    codes, s = k_write.quantize_k(k)
    assert s[0] == 0 and np.all(codes[0] == 0)
    assert s[1] == np.float32(0.5) / np.float32(448.0)
    assert codes[1, 5] == 0xFE and np.count_nonzero(codes[1]) == 1


def test_written_cache_feeds_the_logits_definition():
    """A cache written token by token and read back through the block table
    gives the keys' dequantised values at their logical positions."""
    from oracle import indexer as oi
    rng = np.random.default_rng(11)
    L = 150
    bt = np.array([[4, 0, 2]], dtype=np.int32)
    pos = np.arange(L, dtype=np.int32)
    qsl = np.array([0, L], dtype=np.int32)
    k = rng.standard_normal((L, HEAD_DIM)).astype(np.float32)
    cache = np.zeros((5, PAGE_BYTES), np.uint8)
    k_write.write_k_cache(cache, k, k_write.slot_mapping(bt, qsl, pos))
    codes, s = k_write.quantize_k(k)
    got = oi.gather_k(cache, bt[0], 0, L)
    assert np.array_equal(got, fp8.decode(codes) * s.astype(np.float64)[:, None])
    assert PAGE_KEY_BYTES == 8192


def test_compressed_slot_mapping_by_hand():
    """[HBM] 5.1/5.2: at ratio 4 a 256-token host block stores 64 entries
    (block_size 64), at ratio 128 two; only (p + 1) % ratio == 0 has a slot,
    entry p // ratio, -1 elsewhere."""
    bt = np.array([[3, 7, 12]], dtype=np.int32)
    qsl = np.array([0, 9], dtype=np.int32)
    pos = np.array([0, 2, 3, 7, 255, 256, 259, 511, 767], dtype=np.int32)
    got = k_write.compressed_slot_mapping(bt, qsl, pos, 4, 256 // 4)
    # entries 0, 1, 63, 64 (block 1), 127 (block 1 row 63), 191 (block 2)
    assert list(got) == [-1, -1, 3 * 64 + 0, 3 * 64 + 1, 3 * 64 + 63, -1,
                         7 * 64 + 0, 7 * 64 + 63, 12 * 64 + 63]
    got = k_write.compressed_slot_mapping(bt, qsl, pos, 128, 256 // 128)
    # entries: p = 255 -> 1 (block 0 row 1); 511 -> 3 (block 1 row 1);
    # 767 -> 5 (block 2 row 1)
    assert list(got) == [-1, -1, -1, -1, 3 * 2 + 1, -1, -1, 7 * 2 + 1,
                         12 * 2 + 1]


def test_compressed_slot_mapping_ratio_one_is_plain():
    rng = np.random.default_rng(6)
    bt = rng.permutation(50).astype(np.int32)[:40].reshape(4, 10)
    bt[3, 5:] = -1
    qsl = np.array([0, 30, 30, 70, 100], dtype=np.int32)
    pos = rng.integers(-1, 700, size=100).astype(np.int32)
    assert np.array_equal(
        k_write.compressed_slot_mapping(bt, qsl, pos, 1, PAGE_TOKENS),
        k_write.slot_mapping(bt, qsl, pos))


def test_compressed_positions_brute_force():
    """The last entry all of whose ratio tokens are at or before p, by
    enumeration of entries."""
    for ratio in (1, 2, 3, 4, 128):
        pos = np.arange(-1, 700)
        got = k_write.compressed_positions(pos, ratio)
        for p, g in zip(pos, got):
            seen = [c for c in range(800)
                    if c * ratio + ratio - 1 <= p] if p >= 0 else []
            assert g == (max(seen) if seen else -1), (ratio, p)
    # a boundary token's slot holds exactly the row's last visible entry
    pos = np.array([3, 7, 11, 255], dtype=np.int32)
    assert list(k_write.compressed_positions(pos, 4)) == \
        [int(p) // 4 for p in pos]
