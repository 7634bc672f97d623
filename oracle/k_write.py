"""Indexer-K write path: per-token FP8 quantisation of new keys and their
scatter into the paged cache, plus the slot mapping that addresses them.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (web pages; cited by title and section):

* [KVB] "GLM-5.3 inference pipeline (12): paging budget, prefix hits and
  eviction of the main KV and indexer caches" (pinghaoyang.com.cn).
  - section "the indexer cache's write path": every full layer writes, for
    each new token, its FP8 key and FP32 scale at the token's in-page offset
    (store_quantized(loc, index_k, index_k_scale)); the write volume is
    132 B per token per layer, linear in new tokens; an evicted slot is not
    cleared, the next write overwrites it;
  - section on eviction/reclaim (IndexKeyCache.move comment): a physical
    page stores all key bytes first, then all scale bytes (8448 B for 64
    tokens).
* [HBM] "HBM index architecture design" (vLLM research notes), section 2.3
  (virtual-to-physical translation): slot = block_table[req, pos // 64] * 64
  + pos % 64; section 2.5 (scheduler / worker contract) prints the example
  block row [3, 7, 12]; section 5.1 (DeepSeek-V4 main MLA cache): a
  256-token host block stores 256 // compress_ratio entries (64 at ratio 4,
  2 at ratio 128); section 5.2: the compressed slot mapping.

Readings where the pages are silent (listed in the design doc):
* the key arrives as bf16 [N, 128] (the indexer's projection output, like q)
  and is quantised exactly as q is: amax = max|k|, s = fp32(amax / 448),
  code = e4m3fn(fp32(k / s)); an all-zero key stores s = 0 and zero codes
  (the plain reading of "absmax scale"; q uses s = 1 there, which only
  matters for its own division);
* slot -1 (a padding token) writes nothing;
* two tokens with the same slot in one call are not defined (the write path
  never produces them);
* compressed cache: a row sees the entries whose tokens all lie at or before
  its position (compressed_positions).

Pins: tests/test_oracle_k_write.py -- the [HBM] section 2.5 block row and the
section 2.3 formula on hand positions (golden fixture); the compressed
mapping on hand positions at ratio 4 and 128 (the 5.1 per-block counts) and
its reduction to the plain mapping at ratio 1; the compressed positions
against a brute-force count of fully covered entries; byte offsets of a
hand-built write against the [KVB] page layout, the e4m3 error bound of the
round trip, agreement of the codes with torch's float8_e4m3fn cast (a library
routine), the zero-key and padding-slot cases.
"""

import numpy as np

from . import fp8
from .indexer import (PAGE_TOKENS, HEAD_DIM, PAGE_KEY_BYTES, PAGE_BYTES,
                      request_of_rows)


def slot_mapping(block_table, query_start_loc, positions):
    """Physical slot of every query row's token ([HBM] 2.3):
    block_table[r, p // 64] * 64 + p % 64, or -1 where the block-table entry
    is -1 (no page) or p < 0."""
    bt = np.asarray(block_table, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    req = request_of_rows(query_start_loc, pos.shape[0])
    out = np.full(pos.shape[0], -1, dtype=np.int64)
    for t in range(pos.shape[0]):
        p = int(pos[t])
        if p < 0 or p // PAGE_TOKENS >= bt.shape[1]:
            continue
        page = int(bt[req[t], p // PAGE_TOKENS])
        if page >= 0:
            out[t] = page * PAGE_TOKENS + p % PAGE_TOKENS
    return out


def compressed_slot_mapping(block_table, query_start_loc, positions,
                            compress_ratio, block_size):
    """Slots of a compressed cache ([HBM] 5.2, DeepSeek-V4 compressed slot
    mapping): only a token with (p + 1) % ratio == 0 has a slot; it is entry
    c = p // ratio of its request, stored at block_table[r, c // block_size]
    * block_size + c % block_size (block_size = entries per storage block,
    the host block's tokens // ratio, [HBM] 5.1); every other token gets -1.
    ratio 1 with block_size 64 is ``slot_mapping``."""
    bt = np.asarray(block_table, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    req = request_of_rows(query_start_loc, pos.shape[0])
    out = np.full(pos.shape[0], -1, dtype=np.int64)
    for t in range(pos.shape[0]):
        p = int(pos[t])
        if p < 0 or (p + 1) % compress_ratio != 0:
            continue
        c = p // compress_ratio
        if c // block_size >= bt.shape[1]:
            continue
        blk = int(bt[req[t], c // block_size])
        if blk >= 0:
            out[t] = blk * block_size + c % block_size
    return out


def compressed_positions(positions, compress_ratio):
    """Reading (the pages give no causal rule for compressed entries): a row
    at position p sees entry c when every token it covers, c * ratio ..
    c * ratio + ratio - 1, is at or before p; its position in the compressed
    cache is the last such c, (p + 1) // ratio - 1 (-1: none, or p < 0)."""
    pos = np.asarray(positions, dtype=np.int64)
    out = np.where(pos >= 0, (pos + 1) // compress_ratio - 1, -1)
    return out.astype(np.int64)


def quantize_k(k):
    """Per-token e4m3fn quantisation of k [N, 128] (bf16 values as float32):
    s = fp32(amax / 448), code = e4m3fn(fp32(k / s)); an all-zero token gets
    s = 0 and zero codes.  Returns (codes u8 [N, 128], s f32 [N])."""
    k32 = np.asarray(k, dtype=np.float32)
    assert k32.shape[-1] == HEAD_DIM
    amax = np.max(np.abs(k32), axis=-1)
    s = (amax / np.float32(fp8.E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    x = (k32 / safe[:, None]).astype(np.float32)
    codes = fp8.encode(x)
    codes = np.where((s > 0)[:, None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def write_k_cache(k_cache, k, slots):
    """Store token i's codes and scale at slot slots[i] of ``k_cache``
    (uint8 [num_pages, 8448], modified in place): page slot // 64, row
    slot % 64; key bytes at row * 128, the scale at 8192 + row * 4 ([KVB]).
    Tokens with a negative slot are skipped.  Returns ``k_cache``."""
    codes, s = quantize_k(k)
    slots = np.asarray(slots, dtype=np.int64)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        page, row = int(slot) // PAGE_TOKENS, int(slot) % PAGE_TOKENS
        k_cache[page, row * HEAD_DIM:(row + 1) * HEAD_DIM] = codes[i]
        k_cache[page, PAGE_KEY_BYTES + 4 * row:PAGE_KEY_BYTES + 4 * row + 4] = \
            np.frombuffer(np.float32(s[i]).astype("<f4").tobytes(), np.uint8)
    assert k_cache.shape[1] == PAGE_BYTES
    return k_cache
