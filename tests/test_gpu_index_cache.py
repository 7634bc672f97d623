"""GPU tests of dsa_index_cache_run (IndexCache layer loop) and of the
device-side range checks, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

from dsa_lightning_indexer_amd import binding, synth
from oracle import index_cache as oic
from oracle import indexer as oi
from tests import parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(),
                                 reason="needs a GPU")]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _stack(full_layers, R, context, H, k, seed=3):
    batches = synth.index_cache_layers(full_layers, seed=seed, R=R,
                                       context=context, H=H, k=k)
    ref = batches[full_layers[0]]
    return batches, ref


def _dev_layers(batches, L):
    out = []
    for l in range(L):
        b = batches.get(l)
        out.append(None if b is None else {
            "q_bf16": b.q_bf16.cuda(),
            "weights": torch.from_numpy(b.weights).cuda(),
            "k_cache": torch.from_numpy(b.k_cache).cuda()})
    return out


def _check_run(batches, ref, mask, snaps, k, rows_per_layer=None, dev=None):
    """S snapshots equal the previous F snapshot bit-exactly; F snapshots
    match the oracle (sampled rows: top-k sets and logits) and the
    standalone calls exactly.  ``dev``: device copies of the layers."""
    snaps = snaps.cpu().numpy()
    last_full = None
    bt = torch.from_numpy(ref.block_table).cuda()
    qsl = torch.from_numpy(ref.query_start_loc).cuda()
    pos = torch.from_numpy(ref.positions).cuda()
    for l, s in enumerate(mask):
        if s:
            assert last_full is not None
            assert np.array_equal(snaps[l], snaps[last_full]), f"layer {l}"
            continue
        last_full = l
        b = batches[l]
        lay = dev[l] if dev is not None else {
            "q_bf16": b.q_bf16.cuda(),
            "weights": torch.from_numpy(b.weights).cuda(),
            "k_cache": torch.from_numpy(b.k_cache).cuda()}
        d = dict(lay, block_table=bt, qsl=qsl, positions=pos)
        _, _, lg, tk = parity.run_gpu(b, d, k)
        assert np.array_equal(tk.cpu().numpy(), snaps[l]), \
            f"layer {l}: run() differs from the standalone calls"
        rows = range(b.T) if rows_per_layer is None else rows_per_layer
        rows = list(rows)
        ora = parity.oracle_logits(b, rows=rows)
        mag = parity.magnitude(b, rows=rows)
        lg_rows = lg[rows].cpu().numpy()
        for i, t in enumerate(rows):
            p = int(b.positions[t])
            parity.check_topk_row(snaps[l][t], ora[i, : p + 1], k,
                                  f"layer {l} row {t}")
            parity.check_logits_row(lg_rows[i], ora[i], p,
                                    f"layer {l} row {t}", mag[i])


@pytest.mark.parametrize("cfg", [dict(freq=4, offset=2),
                                 dict(pattern="seeded"),
                                 dict(freq=3, offset=0, mtp=2)])
def test_index_cache_run_reduced(cfg):
    _say(f"case: index cache run reduced {cfg}")
    L = 61
    kw = dict(cfg)
    nh = -1
    if kw.pop("mtp", None):
        nh = L - 2                            # last two layers are MTP
    if kw.get("pattern") == "seeded":
        kw["pattern"] = synth.index_cache_pattern(L)
    mask = binding.dsa_index_cache_mask(L, num_hidden_layers=nh, **kw)
    ref_mask = oic.skip_mask(L, num_hidden_layers=None if nh < 0 else nh, **kw)
    assert mask == ref_mask.tolist()
    if mask[0]:
        with pytest.raises(binding.DsaError):
            binding.dsa_index_cache_run(
                [None] * L, torch.zeros((4, 40), dtype=torch.int32,
                                        device="cuda"),
                torch.arange(5, dtype=torch.int32, device="cuda"),
                torch.zeros(4, dtype=torch.int32, device="cuda"), 2560, 128,
                torch.zeros((4, 128), dtype=torch.int32, device="cuda"),
                num_hidden_layers=nh, H=16, **kw)
        return
    full = [l for l in range(L) if not mask[l]]
    R, context, H, k = 4, 2500, 16, 128
    batches, ref = _stack(full, R, context, H, k)
    buf = torch.full((R + 3, k), 7, dtype=torch.int32, device="cuda")
    calls = []
    skip, snaps = binding.dsa_index_cache_run(
        _dev_layers(batches, L), torch.from_numpy(ref.block_table).cuda(),
        torch.from_numpy(ref.query_start_loc).cuda(),
        torch.from_numpy(ref.positions).cuda(), ref.ld, k, buf,
        num_hidden_layers=nh, snapshots=True,
        callback=lambda layer, is_full: calls.append((layer, is_full)), **kw)
    torch.cuda.synchronize()
    assert skip == mask
    assert calls == [(l, not mask[l]) for l in range(L)]
    assert torch.all(buf[R:] == 7)                 # rows beyond T untouched
    last = max(full)
    assert np.array_equal(buf[:R].cpu().numpy(), snaps[last].cpu().numpy())
    _check_run(batches, ref, mask, snaps, k)
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("rows", [1, 3, 5])
def test_index_cache_run_chunked_equals_unchunked(rows):
    """F layers under a logits budget (rows_per_chunk < T) give every
    layer's buffer rows bit for bit as the unchunked run."""
    _say(f"case: index cache run, {rows} rows per chunk")
    L, R, context, H, k = 9, 6, 1800, 16, 128
    mask = binding.dsa_index_cache_mask(L, freq=2, offset=1)
    full = [l for l in range(L) if not mask[l]]
    batches, ref = _stack(full, R, context, H, k, seed=12)
    dev = _dev_layers(batches, L)
    geo = (torch.from_numpy(ref.block_table).cuda(),
           torch.from_numpy(ref.query_start_loc).cuda(),
           torch.from_numpy(ref.positions).cuda(), ref.ld, k)
    outs = []
    for chunk in (0, rows):
        buf = torch.full((R, k), 3, dtype=torch.int32, device="cuda")
        skip, snaps = binding.dsa_index_cache_run(
            dev, *geo, buf, freq=2, offset=1, snapshots=True,
            rows_per_chunk=chunk)
        torch.cuda.synchronize()
        assert skip == mask
        outs.append(snaps.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_mtp_draft_passes():
    """A trunk pass (4 layers, freq 2), then MTP draft passes over the one
    MTP layer (id 4) through the C ABI: step 0 computes (the oracle's
    top-k of that layer), step 1 with the reuse switch is all S and keeps
    step 0's rows bit-exactly, step 1 without it recomputes the same rows."""
    _say("case: MTP draft passes (trunk freq 2, one MTP layer)")
    nh, R, context, H, k = 4, 4, 2000, 16, 128
    trunk_mask = binding.dsa_index_cache_mask(nh, freq=2, offset=1,
                                              num_hidden_layers=nh)
    full = [l for l in range(nh) if not trunk_mask[l]] + [nh]
    batches, ref = _stack(full, R, context, H, k, seed=8)
    dev = _dev_layers(batches, nh + 1)
    geo = (torch.from_numpy(ref.block_table).cuda(),
           torch.from_numpy(ref.query_start_loc).cuda(),
           torch.from_numpy(ref.positions).cuda(), ref.ld, k)
    buf = torch.full((R, k), 5, dtype=torch.int32, device="cuda")
    skip, _ = binding.dsa_index_cache_run(dev[:nh], *geo, buf, freq=2,
                                          offset=1, num_hidden_layers=nh)
    assert skip == trunk_mask
    calls = []
    skip0, _ = binding.dsa_index_cache_run(
        dev[nh:], *geo, buf, num_hidden_layers=nh, first_layer=nh,
        mtp_draft_step=0, mtp_reuse=True,
        callback=lambda layer, is_full: calls.append((layer, is_full)))
    torch.cuda.synchronize()
    assert skip0 == [False] and calls == [(nh, True)]
    step0 = buf.cpu().numpy().copy()
    b = batches[nh]
    ora = parity.oracle_logits(b)
    for t in range(b.T):
        p = int(b.positions[t])
        parity.check_topk_row(step0[t], ora[t, : p + 1], k, f"mtp row {t}")
    skip1, _ = binding.dsa_index_cache_run(
        [None], *geo, buf, num_hidden_layers=nh, first_layer=nh,
        mtp_draft_step=1, mtp_reuse=True, H=H)
    torch.cuda.synchronize()
    assert skip1 == [True] and np.array_equal(buf.cpu().numpy(), step0)
    buf.fill_(5)
    skip2, _ = binding.dsa_index_cache_run(
        dev[nh:], *geo, buf, num_hidden_layers=nh, first_layer=nh,
        mtp_draft_step=1, mtp_reuse=False)
    torch.cuda.synchronize()
    assert skip2 == [False] and np.array_equal(buf.cpu().numpy(), step0)
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.fixture(scope="module")
def full_stack():
    """The IndexCache workload at full size: 61 layers, each with its own K
    cache, q and weights; 32 decode requests x 16384 context, H = 64, k =
    2048.  Generated once for the three runs below."""
    _say("generating the 61-layer stack (32 x 16384, H=64)")
    L = 61
    batches, ref = _stack(list(range(L)), 32, 16384, 64, 2048)
    dev = _dev_layers(batches, L)
    yield L, batches, ref, dev
    del dev


@pytest.mark.parametrize("run", ["freq4", "pattern", "freq1"])
def test_index_cache_run_full_size(full_stack, run):
    """dsa_index_cache_run at full size with freq 4 / offset 2 (16 F), the
    seeded 61-character pattern and freq 1 (61 F): the mask, S snapshots
    bit-exact, every F layer equal to the standalone calls and 5 oracle rows
    per F layer (top-k sets and logits)."""
    L, batches, ref, dev = full_stack
    kw = {"freq4": dict(freq=4, offset=2),
          "pattern": dict(pattern=synth.index_cache_pattern(L)),
          "freq1": dict(freq=1, offset=2)}[run]
    _say(f"case: index cache full size (61 layers, 32 x 16384), {run}")
    mask = binding.dsa_index_cache_mask(L, **kw)
    assert mask == oic.skip_mask(L, **kw).tolist()
    if run == "freq4":
        assert sum(1 for x in mask if not x) == 16
    if run == "freq1":
        assert not any(mask)
    # layers a run does not compute are passed as None: nothing reads them
    layers = [None if mask[l] else dev[l] for l in range(L)]
    buf = torch.empty((32, 2048), dtype=torch.int32, device="cuda")
    skip, snaps = binding.dsa_index_cache_run(
        layers, torch.from_numpy(ref.block_table).cuda(),
        torch.from_numpy(ref.query_start_loc).cuda(),
        torch.from_numpy(ref.positions).cuda(), ref.ld, 2048, buf,
        snapshots=True, H=64, **kw)
    torch.cuda.synchronize()
    assert skip == mask
    _check_run(batches, ref, mask, snaps, 2048,
               rows_per_layer=[0, 7, 13, 22, 31], dev=dev)
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_out_of_range_block_table_entry_is_flagged_not_faulting():
    """A block_table entry outside the page pool is caught by the kernels'
    bounds check (the address is never formed): its logits are -inf, a
    sticky flag is raised and the rest of the row is unaffected."""
    _say("case: out-of-range block table entry (host-forced)")
    b = synth.tiny()
    d = parity.upload(b)
    binding.dsa_device_error_flags(reset=True)
    for kernel in (0, 1, 2, 4, 5):
        binding.dsa_set_option("logits_kernel", kernel)
        _, _, lg_ok, _ = parity.run_gpu(b, d)     # this kernel, good table
        bad = d["block_table"].clone()
        bad[0, 1] = 1 << 20                       # page id beyond the pool
        d2 = dict(d, block_table=bad)
        _, _, lg, _ = parity.run_gpu(b, d2)
        flags = binding.dsa_device_error_flags(reset=True)
        assert flags & 1
        assert torch.all(torch.isneginf(lg[:, 64:128]))
        assert torch.equal(lg[:, :64], lg_ok[:, :64])
        assert torch.equal(lg[:, 128:256], lg_ok[:, 128:256])
    binding.dsa_set_option("logits_kernel", 0)
    # a position past the logits row is flagged and its row left alone
    pos = d["positions"].clone()
    pos[3] = 10 ** 6
    q8, qs = binding.dsa_quantize_q(d["q_bf16"])
    lg = torch.full((b.T, b.ld), 5.0, device="cuda")
    binding.dsa_indexer_logits(q8, qs, d["weights"], d["k_cache"],
                               d["block_table"], d["qsl"], pos, b.ld, lg)
    assert binding.dsa_device_error_flags(reset=True) & 2
    assert torch.all(lg[3] == 5.0)
