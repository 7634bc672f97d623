"""GPU tests of dsa_indexer_forward (q quantisation, logits and top-k in one
call) through the C ABI: against the separate entry points bit for bit."""

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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _reset():
    binding.dsa_device_error_flags(reset=True)
    yield
    for key in ("logits_kernel", "topk_kernel", "row_pages_per_wave",
                "tile_pages_per_step"):
        binding.dsa_set_option(key, 0)


def _forward(b, d, k=None, **kw):
    k = b.k if k is None else k
    return binding.dsa_indexer_forward(d["q_bf16"], d["weights"], d["k_cache"],
                                       d["block_table"], d["qsl"],
                                       d["positions"], b.ld, k, **kw)


def _batches():
    return {
        "decode64": lambda: synth.decode(),
        "decode100": lambda: synth.decode(R=100),
        "decode_short": lambda: synth.decode(R=24, lo=100, hi=3000, k=256),
        "tiny": lambda: synth.tiny(),
    }


@pytest.mark.parametrize("name", sorted(_batches()))
def test_forward_equals_separate_calls(name):
    _say(f"case: forward vs separate calls, {name}")
    b = _batches()[name]()
    d = parity.upload(b)
    _, _, lg_ref, tk_ref = parity.run_gpu(b, d)
    lg, tk = _forward(b, d)
    torch.cuda.synchronize()
    for t in range(b.T):
        p = int(b.positions[t])
        assert torch.equal(lg[t, : p + 1], lg_ref[t, : p + 1]), f"row {t}"
    assert torch.equal(tk, tk_ref)
    assert binding.dsa_device_error_flags(reset=True) == 0


@pytest.mark.parametrize("H", [20, 48])
def test_forward_partial_heads(H):
    """Head counts that are not a multiple of 16 (padded A rows) and 48."""
    _say(f"case: forward, H={H}")
    b = synth.decode(R=12, H=H, k=512, seed=5)
    d = parity.upload(b)
    lg, tk = _forward(b, d)
    _, _, lg_ref, tk_ref = parity.run_gpu(b, d)
    for t in range(b.T):
        p = int(b.positions[t])
        assert torch.equal(lg[t, : p + 1], lg_ref[t, : p + 1]), f"row {t}"
    assert torch.equal(tk, tk_ref)


def test_forward_repeated_calls_and_workspace_reuse():
    """Dirty workspace, repeated calls, a smaller batch through the same
    workspace: all equal to a fresh call."""
    _say("case: forward repeated calls on one dirty workspace")
    b = synth.decode()
    d = parity.upload(b)
    need = binding.dsa_forward_workspace_size(b.T, b.H, b.ld, b.k)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    lg0, tk0 = _forward(b, d)
    for _ in range(3):
        lg, tk = _forward(b, d, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(tk, tk0)
    small = synth.decode(R=9, seed=31)
    ds = parity.upload(small)
    _, _, _, tk_small_ref = parity.run_gpu(small, ds)
    _, tk_small = _forward(small, ds, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(tk_small, tk_small_ref)


def test_forward_graph_replays():
    """The forward call captured in a HIP graph: every replay equals the
    eager result."""
    _say("case: forward in a HIP graph")
    b = synth.decode()
    d = parity.upload(b)
    need = binding.dsa_forward_workspace_size(b.T, b.H, b.ld, b.k)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    lg = torch.empty((b.T, b.ld), dtype=torch.float32, device="cuda")
    tk = torch.empty((b.T, b.k), dtype=torch.int32, device="cuda")
    _forward(b, d, logits=lg, out=tk, workspace=ws)
    torch.cuda.synchronize()
    ref = tk.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _forward(b, d, logits=lg, out=tk, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            _forward(b, d, logits=lg, out=tk, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        tk.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tk, ref), f"replay {i}"


def test_forward_out_of_range_position_row():
    """A position past the logits row, and one inside it but past the
    request's block-table row: both flagged, their logits rows untouched,
    their top-k rows all -1, every other row as from the separate calls."""
    _say("case: forward with out-of-range positions (host-forced)")
    b = synth.decode(R=16, seed=77)
    d = parity.upload(b)
    _, _, lg_ref, tk_ref = parity.run_gpu(b, d)
    bt_cols = 64 * b.block_table.shape[1]
    ld = bt_cols + 512                       # room for a row past the table
    pos = d["positions"].clone()
    pos[5] = ld + 100                        # past the logits row
    pos[9] = bt_cols + 7                     # inside it, past the table row
    d2 = dict(d, positions=pos)
    lg = torch.full((b.T, ld), 3.0, device="cuda")
    tk = torch.full((b.T, b.k), 11, dtype=torch.int32, device="cuda")
    need = binding.dsa_forward_workspace_size(b.T, b.H, ld, b.k)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    binding.dsa_indexer_forward(d2["q_bf16"], d2["weights"], d2["k_cache"],
                                d2["block_table"], d2["qsl"], pos, ld, b.k,
                                logits=lg, out=tk, workspace=ws)
    torch.cuda.synchronize()
    assert binding.dsa_device_error_flags(reset=True) & 2
    for t in (5, 9):
        assert torch.all(lg[t] == 3.0)
        assert torch.all(tk[t] == -1), f"row {t}"
    keep = [t for t in range(b.T) if t not in (5, 9)]
    assert torch.equal(tk[keep], tk_ref[keep])


@pytest.mark.parametrize("ld,opt", [(4096, 0), (4096, 2), (131072, 0),
                                    (131072, 3)])
def test_topk_position_outside_the_row_gives_minus_one(ld, opt):
    """dsa_indexer_topk: a row at p >= ld (no logits for it) or p < 0 is all
    -1 in every top-k kernel class; a row at ld - 1 is the exact top-k."""
    _say(f"case: top-k rows past ld (ld {ld}, topk_kernel {opt})")
    T, k = 4, 64
    g = torch.Generator().manual_seed(ld + opt)
    logits = torch.randn((T, ld), generator=g).cuda()
    pos = torch.tensor([ld - 1, ld, ld + 1000, -3], dtype=torch.int32,
                       device="cuda")
    out = torch.full((T, k), 11, dtype=torch.int32, device="cuda")
    binding.dsa_set_option("topk_kernel", opt)
    try:
        binding.dsa_indexer_topk(logits, pos, k, out=out)
        torch.cuda.synchronize()
    finally:
        binding.dsa_set_option("topk_kernel", 0)
    out = out.cpu().numpy()
    ref = oi.topk_row(logits[0].cpu().numpy().astype(np.float64), k)
    assert np.array_equal(out[0], np.sort(ref))
    assert np.all(out[1:] == -1)


def test_forward_rejects_small_workspace():
    b = synth.tiny()
    d = parity.upload(b)
    need = binding.dsa_forward_workspace_size(b.T, b.H, b.ld, b.k)
    ws = torch.empty((need - 1,), dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.DsaError) as e:
        _forward(b, d, workspace=ws)
    assert e.value.status == binding.DSA_ERR_WORKSPACE


def _graph_check(run, out, replays=4):
    """Capture run() in a HIP graph on a side stream; every replay (with a
    fill of the output and eager work between replays) equals the eager
    result bit for bit."""
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for i in range(replays):
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        run()                                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"eager after replay {i}"


def test_chunked_forward_graph_replays():
    """The chunked forward (its per-chunk query_start_loc kernel included)
    captured in a HIP graph."""
    _say("case: chunked forward in a HIP graph")
    b = synth.build_batch(np.random.Generator(np.random.PCG64(41)),
                          [3000, 1200], [list(range(2900, 3000)),
                                         list(range(1100, 1200))],
                          H=64, k=256)
    d = parity.upload(b)
    rows = 37
    need = binding.dsa_forward_chunked_workspace_size(b.T, b.R, b.H, b.ld,
                                                      b.k, rows)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    tk = torch.empty((b.T, b.k), dtype=torch.int32, device="cuda")

    def run():
        binding.dsa_indexer_forward_chunked(
            d["q_bf16"], d["weights"], d["k_cache"], d["block_table"],
            d["qsl"], d["positions"], b.ld, b.k, rows_per_chunk=rows, out=tk,
            workspace=ws)
    _graph_check(run, tk)
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_index_cache_run_graph_replays():
    """A five-layer IndexCache run (freq 2, chunked F layers) captured in a
    HIP graph."""
    _say("case: index cache run in a HIP graph")
    L = 5
    mask = binding.dsa_index_cache_mask(L, freq=2, offset=1)
    full = [l for l in range(L) if not mask[l]]
    batches = synth.index_cache_layers(full, seed=17, R=8, context=2000,
                                       H=16, k=128)
    ref = batches[full[0]]
    layers = [None if batches.get(l) is None else {
        "q_bf16": batches[l].q_bf16.cuda(),
        "weights": torch.from_numpy(batches[l].weights).cuda(),
        "k_cache": torch.from_numpy(batches[l].k_cache).cuda()}
        for l in range(L)]
    bt = torch.from_numpy(ref.block_table).cuda()
    qsl = torch.from_numpy(ref.query_start_loc).cuda()
    pos = torch.from_numpy(ref.positions).cuda()
    buf = torch.empty((ref.T, 128), dtype=torch.int32, device="cuda")
    need = binding.dsa_run_workspace_size(ref.T, ref.R, 16, ref.ld, 128, 3)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")

    def run():
        binding.dsa_index_cache_run(layers, bt, qsl, pos, ref.ld, 128, buf,
                                    freq=2, offset=1, rows_per_chunk=3,
                                    workspace=ws)
    _graph_check(run, buf)
    assert binding.dsa_device_error_flags(reset=True) == 0


def test_write_path_and_handoff_graph_replays():
    """Slot mapping, K write, compressed slot mapping and both hand-off
    forms captured in one HIP graph on a side stream (each entry point
    launches on the stream it is given, allocates nothing and records no
    memset): every replay, after the outputs are overwritten and the cache
    restored, equals the eager results."""
    _say("case: write path and hand-off in a HIP graph")
    b = synth.decode(R=8, lo=500, hi=2000, seed=9)
    d = parity.upload(b)
    _, _, _, tk = parity.run_gpu(b, d)
    rng = np.random.default_rng(9)
    kb = torch.from_numpy(rng.standard_normal((b.T, 128)).astype(np.float32)) \
        .bfloat16().cuda()
    cache0 = d["k_cache"].clone()
    slots = torch.empty(b.T, dtype=torch.int64, device="cuda")
    cslots = torch.empty(b.T, dtype=torch.int64, device="cuda")
    cpos = torch.empty(b.T, dtype=torch.int32, device="cuda")
    tslots = torch.empty((b.T, b.k), dtype=torch.int64, device="cuda")
    mask = torch.empty((b.T, b.ld), dtype=torch.float32, device="cuda")

    def calls():
        binding.dsa_slot_mapping(d["block_table"], d["qsl"], d["positions"],
                                 slots=slots)
        binding.dsa_indexer_k_write(kb, slots, d["k_cache"])
        binding.dsa_compressed_slot_mapping(d["block_table"], d["qsl"],
                                            d["positions"], 4, 16,
                                            slots=cslots, positions_c=cpos)
        binding.dsa_topk_to_slots(tk, d["block_table"], d["qsl"], slots=tslots)
        binding.dsa_topk_mask(tk, b.ld, mask=mask)

    outs = (slots, d["k_cache"], cslots, cpos, tslots, mask)
    calls()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d["k_cache"].copy_(cache0)
        calls()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    for i in range(3):
        for x in (slots, cslots, tslots):
            x.fill_(-5)
        cpos.fill_(-5)
        mask.fill_(1.0)
        d["k_cache"].copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (x, r) in enumerate(zip(outs, ref)):
            assert torch.equal(x, r), f"replay {i}, output {j}"
    assert binding.dsa_device_error_flags(reset=True) == 0
