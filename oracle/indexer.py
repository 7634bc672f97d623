"""Lightning-indexer scoring and top-k, written out as plain definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (web pages; cited by title and section):

* [KVB] "GLM-5.3 inference pipeline (12): paging budget, prefix hits and
  eviction of the main KV and indexer caches" (pinghaoyang.com.cn).
  - section "the two caches' byte accounts": the indexer keeps one 128-dim K
    per token, FP8 plus one 4-byte FP32 scale, 132 B per token per layer;
  - section "SGLang: one slot id, two physical buffers": a page holds 64
    tokens; per-layer buffer row = 64 * (128 + 128/128*4) = 8448 bytes;
  - section on eviction/reclaim (IndexKeyCache.move comment): every physical
    page stores all key bytes first, then all scale bytes;
  - section "two costs that are not in pages": shared int32 top-k index buffer
    [max_num_batched_tokens, index_topk]; fp32 logits [rows, cols].
* [HBM] "HBM index architecture design" (vLLM research notes), section 2.3:
  slot = block_table[req, pos // block_size] * block_size + pos % block_size.
* [IC] "vLLM IndexCache practical guide" (blog.gitcode.com), section 2: the
  indexer scores history tokens, clears the shared buffer rows to -1 and
  scatters its top-k there.
* [RFC] "RFC: DeepseekV32 model support" (Ascend msmodeling), section 2.1.3
  "indexer implementation": the indexer path uses FP8 quantisation and an
  fp8_index operator.

The score itself (per-head dot product q_h . k_s, ReLU, sum over heads
weighted by a per-(token, head) weight) is the DeepSeek Sparse Attention
lightning-indexer score (DeepSeek-V3.2, arXiv:2512.02556, which [KVB] lists
among its references).  The pages name the indexer but print no formula or
logit values, so the score formula is PARITY UNPINNED against the pages; it is
pinned against mathematics only (closed forms and invariants in
tests/test_oracle_indexer.py).

Readings where the pages are silent (each listed in the design doc):
* q is quantised per (token, head) to e4m3fn with one absmax/448 fp32 scale
  per 128-element block, the same granularity as K ([KVB], [RFC]);
* dequantised value = code * scale;
* causal bound is inclusive: a query at position p sees tokens 0..p;
* no extra softmax-style scale factor;
* an output index is the token's logical position within its request;
* top-k ties are broken toward the lower index; rows with p+1 <= k list
  0..p and pad with -1.

Pins: tests/test_oracle_indexer.py (brute-force loops on tiny inputs through
byte offsets, closed forms, scale/permutation invariants, layout arithmetic
from [KVB]) and tests/test_oracle_topk.py (k rounds of argmax, padding).
"""

import numpy as np

from . import fp8

PAGE_TOKENS = 64                      # [KVB] 64-token physical pages
HEAD_DIM = 128                        # [KVB] single 128-dim indexer head
QUANT_BLOCK = 128                     # [KVB] one fp32 scale per 128 elements
SCALE_BYTES = HEAD_DIM // QUANT_BLOCK * 4
TOKEN_BYTES = HEAD_DIM + SCALE_BYTES  # 132 B per token per layer
PAGE_KEY_BYTES = PAGE_TOKENS * HEAD_DIM            # 8192: keys first ...
PAGE_BYTES = PAGE_TOKENS * TOKEN_BYTES             # 8448: ... then scales

_DECODE_TABLE = fp8.decode(np.arange(256, dtype=np.uint8))


def quantize_q(q):
    """Quantise q [..., 128] (bf16 values given as float32) per 128-element
    block: amax = max|q|, s = fp32(amax / 448), code = e4m3fn(fp32(q / s)).

    Both divisions are IEEE float32 divisions (numpy float32 arithmetic).  An
    all-zero block gets s = 1 and zero codes.  Returns (codes u8, s f32).
    """
    q32 = np.asarray(q, dtype=np.float32)
    assert q32.shape[-1] == QUANT_BLOCK
    amax = np.max(np.abs(q32), axis=-1)
    s = (amax / np.float32(fp8.E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    x = (q32 / s[..., None]).astype(np.float32)
    return fp8.encode(x), s


def dequantize(codes, scale):
    """code * scale in float64; ``scale`` broadcasts over the last axis."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * \
        np.asarray(scale, dtype=np.float64)[..., None]


def page_keys(k_cache, page):
    """The 64 x 128 key bytes of one physical page (first 8192 bytes)."""
    return k_cache[page, :PAGE_KEY_BYTES].reshape(PAGE_TOKENS, HEAD_DIM)


def page_scales(k_cache, page):
    """The 64 fp32 scales of one physical page (bytes 8192..8447)."""
    raw = np.ascontiguousarray(k_cache[page, PAGE_KEY_BYTES:PAGE_BYTES])
    return raw.view("<f4").astype(np.float32)


def gather_k(k_cache, block_table_row, start, stop):
    """Dequantised K [stop-start, 128] (float64) of logical tokens
    start..stop-1 of one request, through its block-table row ([HBM] 2.3)."""
    s = np.arange(start, stop, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[s // PAGE_TOKENS]
    slots = s % PAGE_TOKENS
    key_off = slots[:, None] * HEAD_DIM + np.arange(HEAD_DIM)[None, :]
    codes = k_cache[pages[:, None], key_off]
    scale_off = PAGE_KEY_BYTES + slots[:, None] * 4 + np.arange(4)[None, :]
    scales = np.ascontiguousarray(k_cache[pages[:, None], scale_off]) \
        .view("<f4").reshape(-1)
    return dequantize(codes, scales)


def request_of_rows(query_start_loc, num_rows):
    """Request index of every query row: r with qsl[r] <= t < qsl[r+1]."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    t = np.arange(num_rows, dtype=np.int64)
    return np.searchsorted(qsl, t, side="right") - 1


def indexer_logits(q_codes, q_scale, weights, k_cache, block_table,
                   query_start_loc, positions, ld, rows=None,
                   token_chunk=32768):
    """Causally masked indexer logits.

    logit[t, s] = sum_h w[t,h] * max(qhat[t,h,:] . khat[s,:], 0) for s <= p_t
    and -inf for s > p_t (columns up to ``ld``).  qhat and khat are the
    dequantised FP8 values (code * scale), all in float64.

    ``rows`` selects a subset of query rows (default: all); the result has
    one row per selected query row.  Work is chunked over tokens only to
    bound memory; each logit is still one sum over 128 dims and one over H.
    """
    T = q_codes.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    req = request_of_rows(query_start_loc, T)
    pos = np.asarray(positions, dtype=np.int64)
    out = np.full((len(rows), ld), -np.inf, dtype=np.float64)
    qhat = {int(t): dequantize(q_codes[t], q_scale[t]) for t in rows}
    w = np.asarray(weights, dtype=np.float64)
    for r in np.unique(req[rows]):
        idx = [i for i, t in enumerate(rows) if req[t] == r]
        n_max = int(max(pos[rows[i]] for i in idx)) + 1
        for a in range(0, n_max, token_chunk):
            b = min(n_max, a + token_chunk)
            khat = gather_k(k_cache, block_table[r], a, b)
            for i in idx:
                t = int(rows[i])
                n = int(pos[t]) + 1
                if a >= n:
                    continue
                e = min(b, n)
                d = qhat[t] @ khat[: e - a].T            # [H, e-a]
                out[i, a:e] = w[t] @ np.maximum(d, 0.0)
    return out


def topk_row(visible, k):
    """Exact top-k of one row's visible logits (positions 0..n-1).

    n <= k: indices 0..n-1 then k-n entries of -1.  Otherwise the first k of
    a stable sort by (logit descending, index ascending).
    """
    v = np.asarray(visible, dtype=np.float64)
    n = v.shape[0]
    if n <= k:
        return np.concatenate([np.arange(n), np.full(k - n, -1)]) \
            .astype(np.int32)
    order = np.lexsort((np.arange(n), -v))
    return order[:k].astype(np.int32)


def indexer_topk(logits, positions, k, rows=None):
    """Top-k of every row of ``logits`` (one row per entry of ``rows``, which
    defaults to all rows), reading only columns 0..p_t."""
    pos = np.asarray(positions, dtype=np.int64)
    rows = np.arange(logits.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), k), dtype=np.int32)
    for i, t in enumerate(rows):
        out[i] = topk_row(logits[i, : int(pos[t]) + 1], k)
    return out


def write_buffer(buffer, topk_rows):
    """Shared-buffer write ([IC] section 2): clear the rows to -1, then store
    the top-k rows.  ``buffer`` is int32 [max_tokens, k], modified in place."""
    T = topk_rows.shape[0]
    buffer[:T] = -1
    buffer[:T, : topk_rows.shape[1]] = topk_rows
    return buffer
