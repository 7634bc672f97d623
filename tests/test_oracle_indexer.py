"""Pins for the oracle's quantisation, paged K gather and logits (CPU only).

Each test checks the oracle against something other than itself: the layout
arithmetic the pages print, the FP8 format's error bound, a pure-Python walk
through raw byte offsets (brute force on tiny inputs), closed forms, and
invariants that a dropped term, a wrong sign, index or transposed operand
would break.
"""

import math
import struct

import numpy as np
import pytest
import torch

from oracle import fp8, indexer
from dsa_lightning_indexer_amd import synth


# ----------------------------------------------------------------- layout --
def test_layout_arithmetic(golden):
    g = golden("layout_arithmetic.json")
    assert indexer.TOKEN_BYTES == g["bytes_per_token_per_layer"] == 132
    assert indexer.PAGE_BYTES == g["bytes_per_page_per_layer"] == 8448
    assert indexer.PAGE_KEY_BYTES == g["key_bytes_per_page"]
    assert indexer.PAGE_TOKENS * (indexer.HEAD_DIM + indexer.HEAD_DIM
                                  // indexer.QUANT_BLOCK * 4) == 8448
    L = g["full_indexer_layers"]
    assert L * indexer.TOKEN_BYTES == g["bytes_per_token_21_layers"]
    assert L * indexer.PAGE_BYTES == g["bytes_per_page_21_layers"]
    assert L * indexer.PAGE_BYTES / 1024 == g["kib_per_page_21_layers"]
    n = g["context_1m_tokens"]
    assert n // indexer.PAGE_TOKENS == g["pages_1m"]
    assert n * L * indexer.TOKEN_BYTES == g["bytes_1m_21_layers"]
    assert n * indexer.TOKEN_BYTES == g["bytes_1m_one_layer"] \
        == g["pages_1m"] * indexer.PAGE_BYTES
    for rows, b in zip(g["topk_buffer_rows"], g["topk_buffer_bytes"]):
        assert rows * g["index_topk"] * 4 == b
    assert n * g["logits_bytes_per_elem"] == g["logits_row_bytes_1m"]


def test_generated_page_layout_matches_byte_walk():
    """Every generated page stores 64 key rows then 64 little-endian fp32
    scales; walk the raw bytes with the slot formula of the vLLM notes
    (slot = block_table[r, pos // 64] * 64 + pos % 64)."""
    b = synth.tiny()
    flat = b.k_cache.reshape(-1)
    khat = indexer.gather_k(b.k_cache, b.block_table[0], 0, 256)
    for pos in [0, 1, 63, 64, 127, 128, 200, 255]:
        slot = int(b.block_table[0, pos // 64]) * 64 + pos % 64
        page, j = divmod(slot, 64)
        base = page * 8448
        key = flat[base + j * 128: base + j * 128 + 128]
        (scale,) = struct.unpack("<f", bytes(flat[base + 8192 + 4 * j:
                                                 base + 8192 + 4 * j + 4]))
        want = [float(fp8.decode(np.uint8(c))) * scale for c in key]
        assert np.array_equal(khat[pos], np.array(want))


# ------------------------------------------------------------ q quantise --
def test_quantize_q_properties():
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((5, 3, 128), dtype=np.float32)
                         * 3).to(torch.bfloat16).float().numpy()
    q[1, 2] = 0.0                                   # amax == 0 block
    q[2, 0, :] = 2.0 ** -130                        # tiny (subnormal) block
    codes, s = indexer.quantize_q(q)
    assert codes.dtype == np.uint8 and s.dtype == np.float32
    assert s[1, 2] == 1.0 and np.all(codes[1, 2] == 0)
    amax = np.abs(q).max(-1)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    # the absmax element lands on code +-448
    for t, h in zip(*np.nonzero(nz)):
        i = int(np.argmax(np.abs(q[t, h])))
        assert fp8.decode(codes[t, h, i]) == math.copysign(448.0, q[t, h, i])
    # FP8 error bound: half an ulp, 2^-4 relative for normals, 2^-10 abs
    # (in units of s) in the subnormal range
    x = q / s[..., None]
    deq = indexer.dequantize(codes, s)
    bound = s[..., None].astype(np.float64) * np.maximum(
        np.abs(x) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - q) <= bound)


def test_quantize_q_encode_step_vs_torch():
    rng = np.random.default_rng(8)
    q = torch.from_numpy(rng.standard_normal((17, 8, 128), dtype=np.float32)) \
        .to(torch.bfloat16).float().numpy()
    codes, s = indexer.quantize_q(q)
    x = (q / s[..., None]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


# ----------------------------------------------------------------- logits --
def _logits_bytewalk(batch, t):
    """Pure-Python fp64 loops over raw bytes for one query row."""
    codes, s = indexer.quantize_q(batch.q_f32)
    H = batch.H
    r = int(np.searchsorted(batch.query_start_loc, t, side="right") - 1)
    p = int(batch.positions[t])
    flat = batch.k_cache.reshape(-1)
    out = []
    for pos in range(p + 1):
        page = int(batch.block_table[r, pos // 64])
        j = pos % 64
        base = page * 8448
        (ks,) = struct.unpack("<f", bytes(flat[base + 8192 + 4 * j:
                                               base + 8192 + 4 * j + 4]))
        kvec = [float(fp8.decode(np.uint8(flat[base + 128 * j + i]))) * ks
                for i in range(128)]
        tot = 0.0
        for h in range(H):
            qs = float(s[t, h])
            d = 0.0
            for i in range(128):
                d += float(fp8.decode(codes[t, h, i])) * qs * kvec[i]
            tot += float(batch.weights[t, h]) * max(d, 0.0)
        out.append(tot)
    return np.array(out)


def _oracle_logits(b, rows=None):
    codes, s = indexer.quantize_q(b.q_f32)
    return indexer.indexer_logits(codes, s, b.weights, b.k_cache,
                                  b.block_table, b.query_start_loc,
                                  b.positions, b.ld, rows=rows)


def test_logits_vs_bytewalk_tiny():
    b = synth.tiny()
    lg = _oracle_logits(b, rows=[0, 7])
    for i, t in enumerate([0, 7]):
        ref = _logits_bytewalk(b, t)
        p = int(b.positions[t])
        np.testing.assert_allclose(lg[i, : p + 1], ref, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(lg[i, p + 1:]))      # causal mask


def test_logits_vs_bytewalk_multi_request():
    rng = np.random.Generator(np.random.PCG64(11))
    b = synth.build_batch(rng, [70, 130, 5], [[69], [64, 129], [0, 4]],
                          H=2, k=8, pool_pages=9)
    lg = _oracle_logits(b)
    for t in range(b.T):
        p = int(b.positions[t])
        np.testing.assert_allclose(lg[t, : p + 1], _logits_bytewalk(b, t),
                                   rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(lg[t, p + 1:]))


def _one_hot_batch(H=1):
    """1 request, 128 tokens; token s's K is c_s * e_{j(s)} with scale 1."""
    rng = np.random.default_rng(5)
    n = 128
    j_of = rng.permutation(128)
    c_codes = rng.integers(0x20, 0x70, size=n).astype(np.uint8)
    c_codes[::3] |= 0x80                             # some negative keys
    bt = np.array([[1, 0]], dtype=np.int32)
    kc = np.zeros((2, 8448), dtype=np.uint8)
    for s in range(n):
        page, slot = bt[0, s // 64], s % 64
        kc[page, slot * 128 + j_of[s]] = c_codes[s]
        kc[page, 8192 + 4 * slot: 8192 + 4 * slot + 4] = \
            np.frombuffer(struct.pack("<f", 1.0), dtype=np.uint8)
    return kc, bt, j_of, c_codes


def test_logits_closed_form_one_hot():
    kc, bt, j_of, c_codes = _one_hot_batch()
    rng = np.random.default_rng(6)
    q = torch.from_numpy(rng.standard_normal((1, 1, 128), dtype=np.float32)) \
        .to(torch.bfloat16).float().numpy()
    codes, s = indexer.quantize_q(q)
    qhat = fp8.decode(codes[0, 0]) * float(s[0, 0])
    lg = indexer.indexer_logits(codes, s, np.ones((1, 1), np.float32), kc, bt,
                                np.array([0, 1], np.int32),
                                np.array([127], np.int32), 256)
    # one nonzero product per key: dot = c_s * qhat[j(s)], logit = ReLU(dot)
    want = np.array([max(fp8.decode(c_codes[t]) * qhat[j_of[t]], 0.0)
                     for t in range(128)])
    assert np.array_equal(lg[0, :128], want)


def test_logits_relu_identity_vs_matmul():
    """logit(q) - logit(-q) = sum_h w_h qhat_h . khat (ReLU(x) - ReLU(-x) = x);
    the right side is one library matmul, independent of the ReLU path."""
    b = synth.tiny()
    codes, s = indexer.quantize_q(b.q_f32)
    ncodes, ns = indexer.quantize_q(-b.q_f32)
    assert np.array_equal(ncodes, codes ^ 0x80) and np.array_equal(ns, s)
    args = (b.weights, b.k_cache, b.block_table, b.query_start_loc,
            b.positions, b.ld)
    lp = indexer.indexer_logits(codes, s, *args)
    ln = indexer.indexer_logits(ncodes, ns, *args)
    khat = indexer.gather_k(b.k_cache, b.block_table[0], 0, 256)
    for t in range(b.T):
        p = int(b.positions[t])
        qhat = indexer.dequantize(codes[t], s[t])            # [H, 128]
        lin = b.weights[t].astype(np.float64) @ (qhat @ khat[: p + 1].T)
        np.testing.assert_allclose(lp[t, : p + 1] - ln[t, : p + 1], lin,
                                   rtol=1e-10, atol=1e-10)
        # and the sum is the weighted |dot|
        ab = b.weights[t].astype(np.float64) @ np.abs(qhat @ khat[: p + 1].T)
        np.testing.assert_allclose(lp[t, : p + 1] + ln[t, : p + 1], ab,
                                   rtol=1e-10, atol=1e-10)


def test_logits_scale_doubling_is_exact():
    b = synth.tiny()
    lg = _oracle_logits(b)
    kc2 = b.k_cache.copy()
    sc = kc2[:, 8192:].copy().view("<f4") * np.float32(2)
    kc2[:, 8192:] = sc.view(np.uint8)
    codes, s = indexer.quantize_q(b.q_f32)
    lg2 = indexer.indexer_logits(codes, s, b.weights, kc2, b.block_table,
                                 b.query_start_loc, b.positions, b.ld)
    fin = np.isfinite(lg)
    assert np.array_equal(lg2[fin], 2 * lg[fin])
    assert np.array_equal(indexer.indexer_topk(lg, b.positions, b.k),
                          indexer.indexer_topk(lg2, b.positions, b.k))


def test_logits_head_permutation_invariant():
    b = synth.tiny()
    lg = _oracle_logits(b)
    perm = np.array([2, 0, 3, 1])
    b2 = synth.IndexerBatch(q_bf16=b.q_bf16[:, perm], weights=b.weights[:, perm],
                            k_cache=b.k_cache, block_table=b.block_table,
                            query_start_loc=b.query_start_loc,
                            positions=b.positions, k=b.k, ld=b.ld)
    np.testing.assert_allclose(_oracle_logits(b2), lg, rtol=1e-12, atol=0)


def test_logits_page_permutation_invariant():
    b = synth.tiny()
    lg = _oracle_logits(b)
    perm = np.array([3, 1, 0, 2])                  # new page of old page i
    kc2 = np.empty_like(b.k_cache)
    kc2[perm] = b.k_cache
    bt2 = perm[b.block_table]
    b2 = synth.IndexerBatch(q_bf16=b.q_bf16, weights=b.weights, k_cache=kc2,
                            block_table=bt2.astype(np.int32),
                            query_start_loc=b.query_start_loc,
                            positions=b.positions, k=b.k, ld=b.ld)
    assert np.array_equal(_oracle_logits(b2), lg)


def test_logits_all_negative_dots_are_zero():
    """If every head's dot is <= 0 the logit is exactly 0 (ReLU)."""
    kc, bt, j_of, c_codes = _one_hot_batch(H=2)
    q = np.zeros((1, 2, 128), np.float32)
    q[0, :, :] = -1.0                         # qhat_j = -1 for every j
    codes, s = indexer.quantize_q(q)
    w = np.array([[0.7, -1.3]], np.float32)
    lg = indexer.indexer_logits(codes, s, w, kc, bt, np.array([0, 1], np.int32),
                                np.array([127], np.int32), 256)
    pos_keys = (c_codes & 0x80) == 0
    assert np.all(lg[0, :128][pos_keys] == 0.0)
    # keys with a negative code give dot = |c| * 448 * s_q > 0 on both heads
    # (q = -1 quantises to code -448 with scale s_q)
    assert np.all(codes == 0xFE)
    neg = ~pos_keys
    w64 = w.astype(np.float64)[0]
    want = np.array([abs(fp8.decode(c)) for c in c_codes[neg]]) * 448.0 * \
        float(s[0, 0]) * (w64[0] + w64[1])
    np.testing.assert_allclose(lg[0, :128][neg], want, rtol=1e-12)
