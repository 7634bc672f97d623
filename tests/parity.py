"""Helpers for the GPU parity tests: upload a synthetic batch, run the HIP
path through the C ABI, and compare with the oracle under the tolerances
stated below.

Tolerances (derived from the arithmetic; both also listed in the design doc):
* logits: |gpu - oracle| <= 2e-3 * |oracle| + 2^-16 * M[t, s] for every
  visible column, where M[t, s] = sum_h |w_th| * sum_i |qhat_thi| |khat_si|
  is the sum of the magnitudes of every product that enters the logit.  The
  relative term is the 2e-3 bound; the absolute term is the summation-error
  bound of the FP8 MFMA's fp32 accumulation (measured on gfx950 at about
  2^-18 of the summed magnitudes per 128-long dot product), which matters
  only where signed head weights cancel and the logit is near 0;
* top-k: same set size, no duplicates, every index in [0, p]; an index in
  the symmetric difference of the GPU and oracle sets is allowed only if its
  oracle logit is within 1e-3 * max(|v_k|, 1e-2 * S_t) of the oracle's k-th
  largest logit v_k (a tie up to the fp32-vs-fp64 difference).
* exactness: the GPU top-k must equal the oracle's top-k applied to the
  GPU's own fp32 logits (same precision decides the same integers), and
  rows with p + 1 <= k must be exactly 0..p then -1.
"""

import numpy as np
import torch

from dsa_lightning_indexer_amd import binding
from oracle import indexer as oi

LOGIT_RTOL = 2e-3
LOGIT_ABS = 2.0 ** -16
LOGIT_FLOOR = 1e-2
TOPK_TIE = 1e-3


# Logits kernel classes the tests force (dsa_set_option "logits_kernel"),
# plus 7: the default tiled kernel with four pages per copy step (the
# instance the launcher picks for grids of more than two rounds).
LOGITS_KERNELS = (0, 1, 2, 3, 4, 5, 6, 7)


def set_logits_kernel(kernel):
    """Force logits kernel class ``kernel`` (0 = automatic)."""
    binding.dsa_set_option("logits_kernel", 6 if kernel == 7 else kernel)
    binding.dsa_set_option("tile_pages_per_step", 4 if kernel == 7 else 0)


def upload(b, device="cuda"):
    d = dict(
        q_bf16=b.q_bf16.to(device),
        weights=torch.from_numpy(b.weights).to(device),
        k_cache=torch.from_numpy(b.k_cache).to(device),
        block_table=torch.from_numpy(b.block_table).to(device),
        qsl=torch.from_numpy(b.query_start_loc).to(device),
        positions=torch.from_numpy(b.positions).to(device),
    )
    return d


def run_gpu(b, d=None, k=None):
    """q quantisation, logits and top-k through the C ABI; host copies."""
    d = upload(b) if d is None else d
    k = b.k if k is None else k
    q8, qs = binding.dsa_quantize_q(d["q_bf16"])
    lg = binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                                    d["block_table"], d["qsl"],
                                    d["positions"], b.ld)
    tk = binding.dsa_indexer_topk(lg, d["positions"], k)
    torch.cuda.synchronize()
    return q8, qs, lg, tk


def _oracle_q(b, rows):
    if rows is None:
        return oi.quantize_q(b.q_f32)
    codes = np.zeros((b.T, b.H, 128), np.uint8)
    s = np.ones((b.T, b.H), np.float32)
    codes[rows], s[rows] = oi.quantize_q(b.q_bf16[rows].float().numpy())
    return codes, s


def oracle_logits(b, rows=None):
    """Oracle logits of ``rows`` (default all); only those rows' q are
    quantised (the others are never read)."""
    rows = None if rows is None else np.asarray(rows, dtype=np.int64)
    codes, s = _oracle_q(b, rows)
    return oi.indexer_logits(codes, s, b.weights, b.k_cache, b.block_table,
                             b.query_start_loc, b.positions, b.ld, rows=rows)


def magnitude(b, rows=None):
    """M[t, s] = sum_h |w_th| sum_i |qhat_thi| |khat_si| (visible columns),
    the scale of the summation error of one logit."""
    rows = np.arange(b.T) if rows is None else np.asarray(rows, np.int64)
    codes, s = _oracle_q(b, rows)
    req = oi.request_of_rows(b.query_start_loc, b.T)
    out = np.zeros((len(rows), b.ld))
    kabs = {}                                  # |khat| of a request's tokens
    for i, t in enumerate(rows):
        p = int(b.positions[t])
        r = int(req[t])
        if r not in kabs or kabs[r].shape[0] < p + 1:
            need = int(max(b.positions[rows][req[rows] == r])) + 1
            kabs[r] = np.abs(oi.gather_k(b.k_cache, b.block_table[r], 0, need))
        qa = np.abs(oi.dequantize(codes[t], s[t]))
        out[i, : p + 1] = np.abs(b.weights[t]).astype(np.float64) @ \
            (qa @ kabs[r][: p + 1].T)
    return out


# The floor criterion (a relative error of at most 2e-3, with a floor for
# logits near zero): |g - o| <= 2e-3 * max(|o|, 1e-2 S_t),
# S_t = max |o| over the row's visible columns.  Every check_logits_row call
# evaluates it on every visible column and appends one record here; the
# session summary (tests/conftest.py) reports the totals.
FLOOR_LOG = []


def floor_ratios(g, o):
    """|g - o| / (2e-3 max(|o|, 1e-2 S_t)) per column (0 where both the
    error and the bound are 0)."""
    o = np.asarray(o, dtype=np.float64)
    err = np.abs(np.asarray(g, dtype=np.float64) - o)
    S = float(np.max(np.abs(o))) if o.size else 0.0
    bound = LOGIT_RTOL * np.maximum(np.abs(o), LOGIT_FLOOR * S)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return r


def check_logits_row(g, o, p, what="", m=None):
    """Logit tolerance on columns 0..p (``m`` = magnitude row; without it
    only the relative term applies).  Also evaluates the floor criterion
    (FLOOR_LOG).  Returns the max relative error over columns with |o| >=
    1e-2 * max|o|."""
    o = np.asarray(o[: p + 1], dtype=np.float64)
    g = np.asarray(g[: p + 1], dtype=np.float64)
    tol = LOGIT_RTOL * np.abs(o)
    if m is not None:
        tol = tol + LOGIT_ABS * np.asarray(m[: p + 1], dtype=np.float64)
    err = np.abs(g - o)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (
        f"{what}: {bad.size} logits out of tolerance, first at s={bad[0]}: "
        f"gpu={g[bad[0]]!r} oracle={o[bad[0]]!r} tol={tol[bad[0]]!r}")
    S = float(np.max(np.abs(o))) if o.size else 0.0
    big = np.abs(o) >= LOGIT_FLOOR * S
    r = floor_ratios(g, o)
    rec = {"what": what, "cols": int(o.size), "viol": int(np.sum(r > 1)),
           "max_ratio": float(r.max()) if r.size else 0.0,
           "viol_cols_max_abs_over_S": float(np.max(np.abs(o[r > 1])) / S)
           if np.any(r > 1) else 0.0}
    if m is not None and np.any(r > 1):
        mm = np.asarray(m[: p + 1], dtype=np.float64)
        rec["viol_max_err_over_M"] = float(np.max(err[r > 1] / mm[r > 1]))
    FLOOR_LOG.append(rec)
    return float(np.max(err[big] / np.abs(o[big]))) if big.any() else 0.0


def check_topk_row(gpu_row, oracle_visible, k, what="", m=None):
    """One GPU top-k row against the oracle's logits: the GPU's set equals
    the oracle's except for indices whose oracle logit lies within the tie
    window of the k-th value (TOPK_TIE relative, floored at LOGIT_FLOOR of
    the row maximum) or, given the magnitude row m, within the two logits'
    combined logits tolerance of it."""
    gpu_row = np.asarray(gpu_row)
    o = np.asarray(oracle_visible, dtype=np.float64)
    n = o.shape[0]
    if n <= k:
        want = np.concatenate([np.arange(n), np.full(k - n, -1)])
        assert np.array_equal(gpu_row, want), f"{what}: padded row differs"
        return 0
    g = gpu_row[:k]
    assert np.all(g >= 0) and np.all(g < n), f"{what}: index out of [0, p]"
    assert np.unique(g).size == k, f"{what}: duplicate indices"
    assert np.all(np.diff(g) > 0), f"{what}: not in ascending order"
    ref = oi.topk_row(o, k)
    diff = np.setxor1d(g, ref)
    if diff.size:
        vk = np.sort(o)[-k]
        S = float(np.max(np.abs(o)))
        win = TOPK_TIE * max(abs(vk), LOGIT_FLOOR * S)
        gap = np.abs(o[diff] - vk)
        if m is not None:
            # two logits closer than the sum of their logits tolerances
            # (LOGIT_RTOL |o| + LOGIT_ABS m) may swap order within the error
            # the logits check permits: such an index is a tie as well
            mm = np.asarray(m[:n], dtype=np.float64)
            kth = int(np.argsort(o, kind="stable")[-k])
            tol = LOGIT_RTOL * np.abs(o) + LOGIT_ABS * mm
            win = np.maximum(win, tol[diff] + tol[kth])
        far = diff[gap > win]
        assert far.size == 0, (
            f"{what}: {far.size} indices differ beyond the tie window "
            f"(first {far[0]}, logit {o[far[0]]!r}, v_k {vk!r})")
    return int(diff.size // 2)


def check_topk_exact_on_gpu_logits(gpu_row, gpu_logits_row, p, k, what=""):
    """GPU top-k == oracle top-k of the GPU's own fp32 logits (sorted)."""
    ref = oi.topk_row(np.asarray(gpu_logits_row[: p + 1], dtype=np.float64), k)
    n = p + 1
    if n <= k:
        assert np.array_equal(np.asarray(gpu_row), ref), what
    else:
        assert np.array_equal(np.asarray(gpu_row), np.sort(ref)), \
            f"{what}: top-k differs from the exact top-k of the GPU logits"
