"""Host logic of bench.py (CPU only): the one-GPU refusal, the counter and
kernel-trace summaries built from rocprofv3 CSV files, and the rule that
byte counters taken for other kernel sources are not reported."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

TILE = ("void dsa::logits_tile16_kernel<1, false, true, 2, true, false>"
        "(dsa::LogitsArgs, int, int, dsa::FusedTile)")
# the fused forward's candidate pass: the same kernel and grid, not the
# forward's logits launch
CAND = ("void dsa::logits_tile16_kernel<1, false, true, 2, true, true>"
        "(dsa::LogitsArgs, int, int, dsa::FusedTile)")
COPY = "__amd_rocclr_copyBuffer"


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                           *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip())["error"]


def _pmc_dir(tmp, name, cal_kib, big, small):
    """Three calibration copies, then logits dispatches at a large grid
    (values ``big``) and a smaller one (``small``); two rows per dispatch
    (the summary adds them)."""
    rows, d = [], 0
    for _ in range(3):
        d += 1
        for half in (0.5, 0.5):
            rows.append(dict(Dispatch_Id=d, Kernel_Name=COPY, Grid_Size=512,
                             Counter_Name="X", Counter_Value=cal_kib * half))
    for grid, vals in ((1 << 20, big), (1 << 16, small)):
        for v in vals:
            d += 1
            for half in (0.25, 0.75):
                rows.append(dict(Dispatch_Id=d, Kernel_Name=TILE,
                                 Grid_Size=grid, Counter_Name="X",
                                 Counter_Value=v * half))
    d += 1
    rows.append(dict(Dispatch_Id=d, Kernel_Name=CAND, Grid_Size=1 << 20,
                     Counter_Name="X", Counter_Value=1e6))
    p = tmp / name
    p.mkdir()
    _write(p / "x_counter_collection.csv", rows)
    return str(p)


def test_pmc_summary_takes_the_largest_grid_and_scales(tmp_path):
    f = _pmc_dir(tmp_path, "f", 131072.0, [100.0, 300.0], [5.0, 5.0, 5.0])
    w = _pmc_dir(tmp_path, "w", 262144.0, [40.0, 40.0], [1.0])
    r = _run("--config", "tiny", "--pmc-summary", f, w)
    assert r.returncode == 0, r.stderr
    d = json.loads(r.stdout)
    assert d["kernel"] == [TILE]
    assert d["fetch_kib_per_dispatch"] == 200.0          # small grid excluded
    assert d["write_kib_per_dispatch"] == 40.0
    assert d["dispatches"] == [2, 2]
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["traffic_bytes_per_launch"] == 200 * 1024 * 2 + 40 * 1024
    assert d["sources_digest"] == bench.logits_sources_digest()
    # every dsa kernel, per (kernel, grid), in the side table
    cand = [e for e in d["every_kernel_per_dispatch"] if e["kernel"] == CAND]
    assert len(cand) == 1 and cand[0]["fetch_kib"] == 1e6


def test_trace_summary_reports_the_workload_launch(tmp_path):
    rows = []
    for grid, durs in (((4096, 4, 1), [1000, 1200, 1100]),
                       ((1024, 1, 1), [100, 100])):
        for dur in durs:
            rows.append(dict(Kernel_Name=TILE, Start_Timestamp=0,
                             End_Timestamp=dur, Grid_Size_X=grid[0],
                             Grid_Size_Y=grid[1], Grid_Size_Z=grid[2]))
    _write(tmp_path / "t_kernel_trace.csv", rows)
    _write(tmp_path / "t_kernel_stats.csv",
           [dict(Name=TILE, Calls=5, AverageNs=700.0, Percentage=100.0)])
    r = _run("--config", "tiny", "--trace-summary", str(tmp_path),
             "--command", "rocprofv3 ... -- python3 bench.py --config tiny")
    assert r.returncode == 0, r.stderr
    out = r.stdout
    assert "rocprofv3 ... -- python3 bench.py --config tiny" in out
    line = [ln for ln in out.splitlines() if ln.startswith("Dominant kernel")]
    assert len(line) == 1
    assert "16384 threads" in line[0] and "3 dispatches" in line[0]
    assert "average 1.100 us" in line[0]


def test_traffic_is_null_once_the_sources_change(tmp_path, monkeypatch):
    p = tmp_path / "c.json"
    monkeypatch.setattr(bench, "counters_path", lambda config: str(p))
    assert bench.traffic_from_counters("decode") is None          # no file
    p.write_text(json.dumps({"sources_digest": "0" * 16,
                             "traffic_bytes_per_launch": 123}))
    assert bench.traffic_from_counters("decode") is None          # stale
    p.write_text(json.dumps({"sources_digest": bench.logits_sources_digest(),
                             "traffic_bytes_per_launch": 123}))
    assert bench.traffic_from_counters("decode") == 123


@pytest.mark.parametrize("config", ["decode", "prefill", "long"])
def test_committed_counters_are_used_only_for_their_sources(config):
    """A committed counter summary names the commands that made it; the
    bench reports its traffic only while the logits kernel sources are the
    ones it was taken on (otherwise null)."""
    with open(bench.counters_path(config)) as f:
        d = json.load(f)
    assert d["commands"], "summary without the commands that made it"
    t = bench.traffic_from_counters(config)
    if d["sources_digest"] == bench.logits_sources_digest():
        assert t == d["traffic_bytes_per_launch"]
    else:
        assert t is None


def test_pmc_summary_refuses_a_foreign_largest_copy(tmp_path):
    """A larger copy than the calibration copies (a timing copy in the
    counter run) would scale every counter wrongly: refused."""
    f = _pmc_dir(tmp_path, "f", 131072.0, [100.0], [])
    rows = list(csv.DictReader(open(os.path.join(f, "x_counter_collection.csv"))))
    rows.append(dict(Dispatch_Id=99, Kernel_Name=COPY, Grid_Size=512,
                     Counter_Name="X", Counter_Value=524288.0))
    _write(tmp_path / "f" / "x_counter_collection.csv", rows)
    w = _pmc_dir(tmp_path, "w", 262144.0, [40.0], [])
    r = _run("--config", "tiny", "--pmc-summary", f, w)
    assert r.returncode != 0
    assert "calibration" in r.stderr


def test_mfma_summary(tmp_path):
    """Multi-counter run: per-dispatch averages of the logits kernel at its
    largest grid only, the busy fraction over GRBM_GUI_ACTIVE x 1024 SIMDs
    and the FP8 work the counters saw (MOPS x 512) against the algorithm's."""
    rows, d = [], 0
    for grid, busy, gui, mops in ((1 << 20, 600.0, 1.0, 10.0),
                                  (1 << 20, 400.0, 1.0, 10.0),
                                  (1 << 16, 1.0, 1.0, 1.0)):
        d += 1
        for name, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                        ("GRBM_GUI_ACTIVE", gui),
                        ("SQ_INSTS_VALU_MFMA_MOPS_F8", mops)):
            rows.append(dict(Dispatch_Id=d, Kernel_Name=TILE, Grid_Size=grid,
                             Counter_Name=name, Counter_Value=v))
    p = tmp_path / "m"
    p.mkdir()
    _write(p / "x_counter_collection.csv", rows)
    r = _run("--config", "tiny", "--mfma-summary", str(p),
             "--command", "rocprofv3 --pmc ... -- python3 bench.py")
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout)
    assert out["dispatches"] == 2
    assert out["counters_per_dispatch"]["SQ_VALU_MFMA_BUSY_CYCLES"] == 500.0
    assert out["xcds"] == 8                      # no agent file: MI355X's
    assert out["mfma_busy_frac"] == round(500.0 / (1.0 / 8 * 1024), 4)
    assert out["counted_fp8_flops"] == 10.0 * 512
    assert out["commands"] == ["rocprofv3 --pmc ... -- python3 bench.py"]


def test_visible_page_ids_match_a_walk_over_the_rows():
    """The bare-read floor reads the pages of every row up to its own
    position, through its own request's block-table row (rows of one
    request repeat its pages, as the logits kernel reads them)."""
    import numpy as np
    from dsa_lightning_indexer_amd import synth
    rng = np.random.Generator(np.random.PCG64(9))
    b = synth.build_batch(rng, [300, 64, 1000, 1], [[299], [0, 63], [],
                                                    [0]], H=4, k=8)
    want = []
    for r in range(b.R):
        for t in range(int(b.query_start_loc[r]),
                       int(b.query_start_loc[r + 1])):
            for j in range(int(b.positions[t]) // 64 + 1):
                want.append(int(b.block_table[r, j]))
    got = bench.visible_page_ids(b)
    assert got.dtype == np.int32 and got.tolist() == want


def test_index_cache_cpu_baseline_runs_the_oracle_stack():
    """The IndexCache CPU leg runs the oracle's layer loop over a freq-4
    stack: on a small stack it completes whole passes and reports rows/s
    for the whole batch."""
    from dsa_lightning_indexer_amd import synth
    from oracle import index_cache as oic
    L = 6
    full = [l for l, s in enumerate(oic.skip_mask(L, freq=4, offset=2))
            if not s]
    host = synth.index_cache_layers(full, R=3, context=300, H=4, k=16,
                                    workers=1)
    ref = host[full[0]]
    rec = bench.cpu_baseline_index_cache(host, ref, L, 0.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "query-rows/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert f"({len(full)} F)" in rec["sample"] and "1 pass(es)" in rec["sample"]
