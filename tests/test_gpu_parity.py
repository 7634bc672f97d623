"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Tolerances are documented in tests/parity.py."""

import sys
import zlib

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import indexer as oi
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _clear_flags():
    binding.dsa_device_error_flags(reset=True)
    yield
    for key in ("logits_kernel", "row_pages_per_wave", "tile_pages_per_split",
                "topk_kernel", "row_head_waves"):
        binding.dsa_set_option(key, 0)


def _assert_no_device_errors():
    assert binding.dsa_device_error_flags(reset=True) == 0


# ------------------------------------------------------------- quantise q --
def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)) \
        .to(torch.bfloat16)


def test_quantize_q_bit_exact():
    _say("case: quantize_q random + special blocks")
    rng = np.random.default_rng(31)
    q = rng.standard_normal((37, 8, 128)).astype(np.float32)
    q[0, 0] = 0.0                                        # amax = 0
    q[0, 1] = 2.0 ** -128                                # subnormal block
    q[1, 0] *= 1e4                                       # large values
    q[1, 1] = 0.0
    q[1, 1, 5] = -3.0                                    # single nonzero
    # amax 448 -> s = 1 exactly; entries at midpoints between FP8 codes
    v = oi.fp8.positive_code_values()
    mids = ((v[:-1] + v[1:]) / 2)[40:126]
    q[2, 0, :] = 0.0
    q[2, 0, 0] = 448.0
    q[2, 0, 1:1 + 60] = mids[:60]
    q[2, 1, :] = 0.0
    q[2, 1, 0] = -448.0
    q[2, 1, 1:1 + 26] = -mids[60:86]
    # the reciprocal path's edges: s just above 2^-100 (amax 2^-91) and
    # just below (amax 2^-92, exact division); a block holding +inf (s =
    # inf: exact division, codes 0 and NaN)
    q[3, 0] *= 2.0 ** -91 / np.abs(q[3, 0]).max()
    q[3, 1] *= 2.0 ** -92 / np.abs(q[3, 1]).max()
    q[3, 2, 7] = np.inf
    qb = _bf16(q)
    q8, qs = binding.dsa_quantize_q(qb.cuda())
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):                  # inf / inf
        codes, s = oi.quantize_q(qb.float().numpy())
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.array_equal(q8.cpu().numpy(), codes)


def test_fp8_code_check_finds_no_mismatch():
    """The q quantisation's fast path (reciprocal with one FMA correction,
    hardware e4m3 conversion) gives the integer encoder's code of the IEEE
    quotient for every pair of bf16 values it is used on, and the hardware
    conversion equals the integer encoder for every fp32 below 464 in
    magnitude: an exhaustive device-side count, no mismatch allowed."""
    _say("case: exhaustive FP8 code check")
    cvt, quotient, codes = binding.dsa_fp8_code_check()
    print(f"fp8 code check: conversion {cvt}, quotient {quotient}, "
          f"codes {codes} mismatches", flush=True)
    assert cvt == 0 and codes == 0


def test_quantize_q_bit_exact_decode_shape():
    _say("case: quantize_q decode batch")
    b = synth.decode()
    q8, qs = binding.dsa_quantize_q(b.q_bf16.cuda())
    torch.cuda.synchronize()
    codes, s = oi.quantize_q(b.q_f32)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.array_equal(q8.cpu().numpy(), codes)


# ------------------------------------------------------------------- tiny --
@pytest.mark.parametrize("kernel", [0, 1, 2, 3, 4, 5])
def test_tiny_logits_and_topk(kernel):
    _say(f"case: tiny, logits kernel option {kernel}")
    binding.dsa_set_option("logits_kernel", kernel)
    b = synth.tiny()
    _, _, lg, tk = parity.run_gpu(b)
    lg, tk = lg.cpu().numpy(), tk.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_logits_row(lg[t], ora[t], p, f"tiny row {t}", mag[t])
        assert np.all(np.isneginf(lg[t, p + 1: (p // 64 + 1) * 64]))
        parity.check_topk_row(tk[t], ora[t, : p + 1], b.k, f"tiny row {t}")
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t], p, b.k)
    _assert_no_device_errors()


# ----------------------------------------------------------------- decode --
@pytest.mark.parametrize("kernel", [0, 2, 3, 4])
def test_decode_batch_all_rows(kernel):
    _say(f"case: decode batch (64 x U[1024,8192], H=64, k=2048), kernel {kernel}")
    binding.dsa_set_option("logits_kernel", kernel)
    b = synth.decode()
    _, _, lg, tk = parity.run_gpu(b)
    lg, tk = lg.cpu().numpy(), tk.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    worst = 0.0
    err_m = 0.0
    padded = 0
    for t in range(b.T):
        p = int(b.positions[t])
        worst = max(worst, parity.check_logits_row(lg[t], ora[t], p,
                                                   f"decode row {t}", mag[t]))
        parity.check_topk_row(tk[t], ora[t, : p + 1], b.k, f"decode row {t}")
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t], p, b.k)
        padded += p + 1 <= b.k
        err_m = max(err_m, float(np.max(np.abs(lg[t, : p + 1] - ora[t, : p + 1])
                                        / mag[t, : p + 1])))
    _say(f"decode max rel logit err (|o| >= 1e-2 max) {worst:.3e}, "
         f"max |err| / M = {err_m:.3e} (2^{np.log2(err_m):.1f}), "
         f"padded rows {padded}")
    assert padded > 0                 # the batch exercises -1 padding
    _assert_no_device_errors()


@pytest.mark.parametrize("hw", [0, 2, 4, 8])
def test_decode_head_waves(hw):
    """Head waves on each row's first pages (option value 1 + their number;
    0 = the default one): logits bit-identical to the balanced kernel
    without them (value 1; same per-page arithmetic), top-k too; also with
    several rows per request (the request guess fails)."""
    _say(f"case: decode with head-wave option {hw}")
    for b in (synth.decode(R=64, lo=100, hi=3000, seed=31),
              synth.build_batch(np.random.Generator(np.random.PCG64(8)),
                                [900, 2000, 40],
                                [[899, 500, 3], [1999, 1000, 77, 64], [39]],
                                H=64, k=256)):
        binding.dsa_set_option("row_head_waves", 1)            # none
        _, _, lg0, tk0 = parity.run_gpu(b)
        binding.dsa_set_option("row_head_waves", hw)
        _, _, lg1, tk1 = parity.run_gpu(b)
        for t in range(b.T):
            p = int(b.positions[t])
            assert torch.equal(lg0[t, : p + 1], lg1[t, : p + 1]), f"row {t}"
        assert torch.equal(tk0, tk1)
        ora = parity.oracle_logits(b, rows=[0, b.T - 1])
        mag = parity.magnitude(b, rows=[0, b.T - 1])
        lg1h = lg1.cpu().numpy()
        for i, t in enumerate([0, b.T - 1]):
            parity.check_logits_row(lg1h[t], ora[i], int(b.positions[t]),
                                    f"row {t}", mag[i])
    _assert_no_device_errors()


@pytest.mark.parametrize("rows", [100, 128])
def test_decode_batch_two_position_chunks(rows):
    """More than 64 decode rows: the balanced row kernel reads the positions
    in two chunks of 64 lanes."""
    _say(f"case: decode batch of {rows} rows")
    b = synth.decode(R=rows)
    _, _, lg, tk = parity.run_gpu(b)
    lg, tk = lg.cpu().numpy(), tk.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_logits_row(lg[t], ora[t], p, f"decode row {t}", mag[t])
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t], p, b.k)
    _assert_no_device_errors()


# ---------------------------------------------------------------- prefill --
@pytest.mark.parametrize("kernel", [0, 5])
def test_prefill_chunk_sampled_rows(kernel):
    _say(f"case: prefill chunk (8192 q x 40960 ctx, H=64, k=2048), "
         f"logits kernel {kernel}")
    binding.dsa_set_option("logits_kernel", kernel)
    b = synth.prefill()
    _, _, lg, tk = parity.run_gpu(b)
    rng = np.random.default_rng(2)
    # 256 evenly spaced rows (the sample the bench's CPU leg times) plus the
    # tile and page edges
    even = np.linspace(0, b.T - 1, 256).round().astype(np.int64).tolist()
    rows = sorted(set([0, 1, 15, 16, 17, 63, 64, 4095, 8190, 8191] + even))
    ora = parity.oracle_logits(b, rows=rows)
    mag = parity.magnitude(b, rows=rows)
    lg_rows = lg[rows].cpu().numpy()
    tk_all = tk.cpu().numpy()
    for i, t in enumerate(rows):
        p = int(b.positions[t])
        parity.check_logits_row(lg_rows[i], ora[i], p, f"prefill row {t}",
                                mag[i])
        parity.check_topk_row(tk_all[t], ora[i, : p + 1], b.k,
                              f"prefill row {t}")
        parity.check_topk_exact_on_gpu_logits(tk_all[t], lg_rows[i], p, b.k)
    # every row: k distinct ascending indices within [0, p]
    assert np.all(tk_all >= 0)
    assert np.all(np.diff(tk_all, axis=1) > 0)
    assert np.all(tk_all.max(axis=1) <= b.positions)
    # exact top-k of the GPU logits on a wider sample of rows
    more = rng.choice(b.T, 64, replace=False)
    lg_more = lg[torch.from_numpy(np.sort(more)).cuda()].cpu().numpy()
    for i, t in enumerate(np.sort(more)):
        parity.check_topk_exact_on_gpu_logits(tk_all[t], lg_more[i],
                                              int(b.positions[t]), b.k)
    _assert_no_device_errors()


# ----------------------------------------------------------- long context --
@pytest.mark.parametrize("kernel", [0, 5])
def test_long_context_rows(kernel):
    _say(f"case: long context (1M tokens, 16 rows, H=64, k=2048), "
         f"logits kernel {kernel}")
    binding.dsa_set_option("logits_kernel", kernel)
    b = synth.long_context()
    _, _, lg, tk = parity.run_gpu(b)
    tk = tk.cpu().numpy()
    # every row of the default kernel against the oracle; four of the
    # alternative epilogue's
    rows = list(range(b.T)) if kernel == 0 else [0, 5, 10, 15]
    ora = parity.oracle_logits(b, rows=rows)
    mag = parity.magnitude(b, rows=rows)
    for i, t in enumerate(rows):
        p = int(b.positions[t])
        g = lg[t, : p + 1].cpu().numpy()
        parity.check_logits_row(g, ora[i], p, f"long row {t}", mag[i])
        parity.check_topk_row(tk[t], ora[i, : p + 1], b.k, f"long row {t}")
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t].cpu().numpy(), p,
                                              b.k, f"long row {t}")
    _assert_no_device_errors()


# ------------------------------------------------------------- edge cases --
def _edge_batch(seed, contexts, positions, H, k, **kw):
    rng = np.random.Generator(np.random.PCG64(seed))
    return synth.build_batch(rng, contexts, positions, H=H, k=k, **kw)


EDGE_CASES = {
    "single_page": ([40], [[39]], 8, 16),
    "one_token": ([1], [[0]], 4, 1),
    "k1": ([300], [[299]], 16, 1),
    "page_edges": ([127, 128, 129, 64, 63, 65], [[126], [127], [128], [63],
                                                [62], [64]], 32, 64),
    "context_below_k": ([100, 3000], [[99], [2999]], 64, 2048),
    "h20_multi_rows": ([700, 333], [list(range(650, 700)),
                                    [0, 1, 2, 100, 332]], 20, 96),
    "ragged_prefill": ([1000], [list(range(0, 1000, 7))], 64, 128),
}


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
@pytest.mark.parametrize("kernel", [1, 2, 3, 4, 5, 6, 7])
def test_edge_cases(name, kernel):
    _say(f"case: edge {name}, logits kernel {kernel}")
    parity.set_logits_kernel(kernel)
    contexts, positions, H, k = EDGE_CASES[name]
    b = _edge_batch(zlib.crc32(name.encode()) % 1000, contexts, positions, H, k,
                    pool_pages=sum((c + 63) // 64 for c in contexts) + 3)
    _, _, lg, tk = parity.run_gpu(b)
    lg, tk = lg.cpu().numpy(), tk.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_logits_row(lg[t], ora[t], p, f"{name} row {t}", mag[t])
        parity.check_topk_row(tk[t], ora[t, : p + 1], k, f"{name} row {t}")
        parity.check_topk_exact_on_gpu_logits(tk[t], lg[t], p, k)
    _assert_no_device_errors()


def test_empty_batch_is_noop():
    _say("case: T = 0")
    d = torch.empty(0, 4, 128, dtype=torch.bfloat16, device="cuda")
    q8, qs = binding.dsa_quantize_q(d)
    assert q8.shape == (0, 4, 128)
    lg = torch.empty(0, 256, device="cuda")
    tk = binding.dsa_indexer_topk(lg, torch.empty(0, dtype=torch.int32,
                                                  device="cuda"), 8)
    assert tk.shape == (0, 8)


def test_page_permutation_gives_identical_logits():
    _say("case: page permutation invariance")
    b = synth.decode(R=8)
    perm = np.random.default_rng(9).permutation(b.k_cache.shape[0])
    kc2 = np.empty_like(b.k_cache)
    kc2[perm] = b.k_cache
    bt2 = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1)
    b2 = synth.IndexerBatch(q_bf16=b.q_bf16, weights=b.weights, k_cache=kc2,
                            block_table=bt2.astype(np.int32),
                            query_start_loc=b.query_start_loc,
                            positions=b.positions, k=b.k, ld=b.ld)
    _, _, lg1, tk1 = parity.run_gpu(b)
    _, _, lg2, tk2 = parity.run_gpu(b2)
    for t in range(b.T):
        p = int(b.positions[t])
        assert torch.equal(lg1[t, : p + 1], lg2[t, : p + 1])
    assert torch.equal(tk1, tk2)


@pytest.mark.parametrize("kernel", [1, 2, 4])
def test_topk_ties_and_constant_rows(kernel):
    _say(f"case: top-k ties, top-k kernel {kernel}")
    binding.dsa_set_option("topk_kernel", kernel)
    T, ld, k = 6, 4096, 100
    rng = np.random.default_rng(12)
    lg = rng.integers(-4, 5, size=(T, ld)).astype(np.float32)
    lg[1] = 1.5                                           # constant row
    lg[2, ::2] = -0.0                                     # -0 vs +0
    lg[2, 1::2] = 0.0
    lg[3] = rng.standard_normal(ld).astype(np.float32)
    lg[3, 17] = np.inf
    pos = np.array([4095, 3000, 999, 4095, 50, 2047], np.int32)
    g = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                 torch.from_numpy(pos).cuda(), k).cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lg[t], int(pos[t]), k,
                                              f"ties row {t}")


@pytest.mark.parametrize("kernel", [1, 2, 4])
@pytest.mark.parametrize("ld", [256, 4096, 8192, 20480, 40960, 49152, 53248])
def test_topk_row_lengths(ld, kernel):
    """Single-workgroup top-k over row lengths that span one to twelve
    4096-column slices (and one past the register-resident limit), with
    random, integer-tied and constant rows, rows just above and below k,
    and a row whose length is the whole ld."""
    _say(f"case: top-k rows of ld {ld}, top-k kernel {kernel}")
    binding.dsa_set_option("topk_kernel", kernel)
    k = 2048 if ld >= 4096 else 64
    rng = np.random.default_rng(ld + kernel)
    T = 8
    lg = (rng.standard_normal((T, ld)) * 5).astype(np.float32)
    lg[1] = np.round(lg[1])                            # many ties
    lg[2] = -3.25                                      # constant
    lg[5, : ld // 2] = -np.inf
    pos = np.array([ld - 1, ld - 1, ld // 2, k, k - 1, ld - 1,
                    min(ld - 1, k + 4097), max(0, ld - 4093)], np.int32)
    g = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                 torch.from_numpy(pos).cuda(), k).cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lg[t], int(pos[t]), k,
                                              f"ld {ld} row {t}")


@pytest.mark.parametrize("kernel", [1, 2, 4])
@pytest.mark.parametrize("ld", [4096, 8192, 16384])
def test_topk_threshold_among_huge_negative_logits(ld, kernel):
    """Rows whose k-th largest logit is below -2^96 or -inf, so the bin it
    falls in is one of the lowest 256 of the first pass and the second and
    third passes run: distinct huge negative values, values that agree in
    their top 24 key bits, -inf with a few finite values, and negative
    values in a band narrower than a first-pass bin."""
    _say(f"case: top-k threshold among huge negative logits, ld {ld}, "
         f"top-k kernel {kernel}")
    binding.dsa_set_option("topk_kernel", kernel)
    k = 2048
    rng = np.random.default_rng(ld + 7 * kernel)
    T = 6
    lg = np.empty((T, ld), np.float32)
    lg[0] = -(1e30 * (1.0 + rng.random(ld))).astype(np.float32)
    lg[0, : k // 2] = rng.standard_normal(k // 2)      # fewer than k finite
    base = np.float32(-3e30).view(np.uint32)
    lg[1] = (base + rng.integers(0, 256, ld).astype(np.uint32)).view(
        np.float32)                                    # one 24-bit prefix
    lg[1, ::5] = rng.standard_normal(len(lg[1, ::5]))
    lg[2] = -np.inf
    lg[2, rng.choice(ld, k // 4, replace=False)] = 1.0
    lg[3] = -np.inf
    lg[4] = -(2.0 ** 100) * (1.0 + rng.random(ld) * 1e-3).astype(np.float32)
    lg[5] = -(1e35 * rng.random(ld)).astype(np.float32)
    pos = np.array([ld - 1, ld - 1, ld - 1, ld - 1, ld - 2, ld - 1], np.int32)
    g = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                 torch.from_numpy(pos).cuda(), k).cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lg[t], int(pos[t]), k,
                                              f"huge negative row {t}")


@pytest.mark.parametrize("kernel", [0, 1])
@pytest.mark.parametrize("k", [512, 2048])
def test_topk_rows_looped_per_workgroup(k, kernel):
    """More rows than compute units: each resident workgroup takes several
    rows in turn with the next row's keys prefetched, so consecutive rows of
    one workgroup mix random, tied, constant, short (<= k) and empty rows.
    k = 512 of 8192 columns takes the column-bitmap emit, k = 2048 the
    per-slice one."""
    _say(f"case: top-k, 700 rows looped over resident workgroups, k={k}, "
         f"top-k kernel {kernel}")
    binding.dsa_set_option("topk_kernel", kernel)
    T, ld = 700, 8192
    rng = np.random.default_rng(k)
    lg = (rng.standard_normal((T, ld)) * 3).astype(np.float32)
    kind = np.arange(T) % 5
    lg[kind == 1] = np.round(lg[kind == 1])                 # many ties
    lg[kind == 2] = 0.75                                    # constant
    pos = rng.integers(k + 1, ld, size=T).astype(np.int32)
    pos[kind == 3] = rng.integers(0, k + 1, size=int((kind == 3).sum()))
    pos[np.arange(T) % 97 == 5] = -1                        # empty rows
    g = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                 torch.from_numpy(pos).cuda(), k).cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lg[t], int(pos[t]), k,
                                              f"looped row {t}")


def test_topk_unaligned_logits_rows():
    """A logits pointer that is not 16-byte aligned takes the LDS-cached
    kernel; results are the exact top-k either way."""
    _say("case: top-k on an unaligned logits view")
    T, ld, k = 4, 4096, 512
    rng = np.random.default_rng(5)
    base = torch.from_numpy(rng.standard_normal(T * ld + 1)
                            .astype(np.float32)).cuda()
    lg = base[1:].view(T, ld)
    pos = torch.tensor([4095, 2000, 600, 511], dtype=torch.int32,
                       device="cuda")
    g = binding.dsa_indexer_topk(lg, pos, k).cpu().numpy()
    lgh = lg.cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lgh[t], int(pos[t]), k,
                                              f"unaligned row {t}")


@pytest.mark.parametrize("kernel", [0, 3])
def test_topk_multi_workgroup_rows(kernel):
    """Rows in a batch wider than 65536 columns: sample select (0) or the
    multi-workgroup radix select (3).  Long, mid-length, short (padded) and
    constant rows (candidate overflow -> exact fallback), heavy near-ties,
    a row whose top keys sit in one narrow run of columns, a row of -inf
    with a few finite keys."""
    _say(f"case: long-row top-k, kernel {kernel}")
    binding.dsa_set_option("topk_kernel", kernel)
    T, ld, k = 10, 131072, 2048
    rng = np.random.default_rng(44)
    lg = rng.standard_normal((T, ld)).astype(np.float32)
    lg[1] = 0.5                                   # all equal: overflow path
    lg[3, :1000] = rng.integers(-2, 3, 1000)      # short row with ties
    lg[4] = np.round(lg[4] * 4) / 4               # heavy near-ties
    lg[6, 50000:52100] += 30.0                    # answer in one narrow run
    lg[7] = -np.inf
    lg[7, rng.choice(ld, 3000, replace=False)] = rng.standard_normal(3000)
    pos = np.array([ld - 1, 90000, 70000, 999, ld - 1, 65536, ld - 1, ld - 1,
                    10000, 20000], np.int32)
    assert binding.dsa_topk_workspace_size(T, ld, k) > 0
    g = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                 torch.from_numpy(pos).cuda(), k).cpu().numpy()
    for t in range(T):
        parity.check_topk_exact_on_gpu_logits(g[t], lg[t], int(pos[t]), k,
                                              f"multi-wg row {t}")
