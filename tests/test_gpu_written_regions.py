"""What each entry point writes and what it leaves alone, as the header
states it: a logits row t (position p) gets values on columns 0..p, -inf on
p < s < 64 ceil((p + 1) / 64) and nothing after that, whatever the other
rows of its tile reach; a top-k row gets slots 0..k-1 only.  Every logits
kernel class is forced in turn, on one row per request (decode) and on many
rows per request at scattered positions (tiles whose rows end on different
pages), with spare columns and spare output slots pre-filled."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import indexer as oi
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]

SENTINEL = 7.25
SLOT_SENTINEL = -77


@pytest.fixture(autouse=True)
def _reset():
    binding.dsa_device_error_flags(reset=True)
    yield
    parity.set_logits_kernel(0)
    binding.dsa_set_option("topk_kernel", 0)


def _batch(layout):
    rng = np.random.Generator(np.random.PCG64(4242 if layout == "decode"
                                              else 4343))
    if layout == "decode":
        ctx = rng.integers(1, 1500, 20).tolist()
        pos = [[L - 1] for L in ctx]
    else:
        # rows of one request in any order, spanning many pages: a 16-row
        # tile holds rows that end on different pages
        ctx = [1900, 700, 64]
        pos = [rng.integers(0, 1900, 37).tolist(),
               rng.integers(0, 700, 21).tolist(),
               [63, 0, 31]]
    b = synth.build_batch(rng, ctx, pos, H=16, k=100)
    b.ld += 512                                   # spare columns
    return b


@pytest.mark.parametrize("layout", ["decode", "scattered"])
@pytest.mark.parametrize("kernel", parity.LOGITS_KERNELS)
def test_logits_written_region(layout, kernel):
    b = _batch(layout)
    print(f"case: layout {layout} logits_kernel {kernel} T={b.T} ld={b.ld}",
          flush=True)
    sys.stdout.flush()
    parity.set_logits_kernel(kernel)
    d = parity.upload(b)
    q8, qs = binding.dsa_quantize_q(d["q_bf16"])
    lg = torch.full((b.T, b.ld), SENTINEL, dtype=torch.float32, device="cuda")
    binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                               d["block_table"], d["qsl"], d["positions"],
                               b.ld, logits=lg)
    torch.cuda.synchronize()
    g = lg.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        p = int(b.positions[t])
        end = 64 * ((p + 1 + 63) // 64)
        parity.check_logits_row(g[t], ora[t], p, f"row {t}", mag[t])
        assert np.all(np.isneginf(g[t, p + 1:end])), f"row {t}: tail of page"
        assert np.all(g[t, end:] == SENTINEL), f"row {t}: column past its pages"
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("topk_kernel", [0, 1, 2, 4])
def test_topk_writes_only_k_slots(topk_kernel):
    b = _batch("scattered")
    print(f"case: topk_kernel {topk_kernel} T={b.T}", flush=True)
    binding.dsa_set_option("topk_kernel", topk_kernel)
    d = parity.upload(b)
    _, _, lg, ref = parity.run_gpu(b, d)
    spare = 40
    out = torch.full((b.T, b.k + spare), SLOT_SENTINEL, dtype=torch.int32,
                     device="cuda")
    binding.dsa_indexer_topk(lg, d["positions"], b.k, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[:, : b.k], ref.cpu().numpy())
    assert np.all(o[:, b.k:] == SLOT_SENTINEL)
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("topk_kernel", [0, 3])
def test_long_row_topk_writes_only_k_slots(topk_kernel):
    """Rows longer than 65536 columns (sample select, 0; multi-workgroup
    radix, 3) into a wider buffer: the exact top-k in slots 0..k-1, nothing
    after; a short row of the same batch is padded."""
    rng = np.random.default_rng(99)
    ld, k, spare = 70144, 2048, 40
    pos = np.array([70000, 65600, 1000, ld - 1], dtype=np.int32)
    T = pos.size
    lg = rng.standard_normal((T, ld)).astype(np.float32)
    print(f"case: long rows, topk_kernel {topk_kernel}", flush=True)
    binding.dsa_set_option("topk_kernel", topk_kernel)
    out = torch.full((T, k + spare), SLOT_SENTINEL, dtype=torch.int32,
                     device="cuda")
    binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                             torch.from_numpy(pos).cuda(), k, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for t in range(T):
        want = oi.topk_row(lg[t, : pos[t] + 1], k)
        want = np.concatenate([np.sort(want[want >= 0]), want[want < 0]])
        assert np.array_equal(o[t, :k], want), f"row {t}"
    assert np.all(o[:, k:] == SLOT_SENTINEL)
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("topk_kernel,ld", [(0, 8192), (1, 8192), (2, 8192),
                                            (4, 8192), (0, 70144),
                                            (3, 70144)])
def test_topk_reads_only_columns_up_to_p(topk_kernel, ld):
    """Columns past a row's position hold values that would win the
    selection (1e30, +inf): every top-k kernel class ignores them."""
    rng = np.random.default_rng(ld + topk_kernel)
    k = 300
    pos = np.array([ld - 1, ld // 2 + 7, 5000, 299, 300, 0], dtype=np.int32)
    T = pos.size
    lg = rng.standard_normal((T, ld)).astype(np.float32)
    for t in range(T):
        lg[t, pos[t] + 1:] = np.float32(1e30)
        lg[t, pos[t] + 1::7] = np.inf
    print(f"case: columns past p, topk_kernel {topk_kernel}, ld {ld}",
          flush=True)
    binding.dsa_set_option("topk_kernel", topk_kernel)
    out = binding.dsa_indexer_topk(torch.from_numpy(lg).cuda(),
                                   torch.from_numpy(pos).cuda(), k)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for t in range(T):
        want = oi.topk_row(lg[t, : pos[t] + 1], k)
        want = np.concatenate([np.sort(want[want >= 0]), want[want < 0]])
        assert np.array_equal(o[t], want), f"row {t}"
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("layout", ["decode", "scattered"])
@pytest.mark.parametrize("kernel", parity.LOGITS_KERNELS)
def test_logits_ignore_block_table_entries_past_the_rows(layout, kernel):
    """Block-table entries past the last page a request's rows reach hold
    an out-of-pool page id: no kernel uses them (no range flag, logits as
    with a clean table)."""
    b = _batch(layout)
    b.block_table = np.concatenate(
        [b.block_table, np.full((b.R, 3), -1, np.int32)], axis=1)
    qsl = b.query_start_loc
    for r in range(b.R):
        rows = b.positions[qsl[r]:qsl[r + 1]]
        need = (int(rows.max()) + 64) // 64 if rows.size else 0
        b.block_table[r, need:] = 1 << 30
    print(f"case: junk past the pages, layout {layout}, kernel {kernel}",
          flush=True)
    parity.set_logits_kernel(kernel)
    _, _, lg, _ = parity.run_gpu(b)
    assert binding.dsa_device_error_flags(reset=True) == 0
    g = lg.cpu().numpy()
    ora = parity.oracle_logits(b)
    mag = parity.magnitude(b)
    for t in range(b.T):
        parity.check_logits_row(g[t], ora[t], int(b.positions[t]), f"row {t}",
                                mag[t])
