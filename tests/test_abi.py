"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/dsa_indexer.h declares, and rejects bad arguments on the host before
touching the device.  Host-only entry points (mask, sizes, options) run."""

import ctypes
import os
import re

import pytest

from dsa_lightning_indexer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dsa_[a-z_0-9]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["dsa_indexer_logits", "dsa_indexer_topk", "dsa_index_cache_run",
                 "dsa_index_cache_mask", "dsa_quantize_q", "dsa_last_error"]:
        assert must in names


def test_every_declared_symbol_is_exported():
    L = binding.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(binding._SIGNATURES)


def test_version_and_last_error():
    L = binding.lib()
    assert L.dsa_version() >= 100
    assert isinstance(L.dsa_last_error(), bytes)


def test_mask_via_abi_matches_pages_example(golden):
    g = golden("index_cache_examples.json")
    m = binding.dsa_index_cache_mask(61, freq=4, offset=2)
    assert [i for i, s in enumerate(m) if not s] == \
        g["freq4_offset2_61"]["full_layers"]
    p = g["pattern_61"]["pattern"]
    m = binding.dsa_index_cache_mask(61, pattern=p, freq=4, offset=2)
    assert [i for i, s in enumerate(m) if not s] == g["pattern_61"]["full_layers"]
    assert not any(binding.dsa_index_cache_mask(61))           # defaults
    m = binding.dsa_index_cache_mask(64, pattern="F" + "S" * 63,
                                     num_hidden_layers=61)
    assert all(m[1:61]) and not any(m[61:])
    assert binding.dsa_index_cache_mask(5, pattern="FS") == \
        [False, True, False, False, False]


@pytest.mark.parametrize("kw", [dict(freq=0), dict(pattern="FFX"),
                                dict(pattern="fs"), dict(freq=-3)])
def test_mask_rejects_bad_config(kw):
    with pytest.raises(binding.DsaError) as e:
        binding.dsa_index_cache_mask(8, **kw)
    assert e.value.status == binding.DSA_ERR_INVALID_ARG


def test_mask_matches_oracle_on_many_configs():
    from oracle import index_cache
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        L = int(rng.integers(0, 80))
        freq = int(rng.integers(1, 9))
        off = int(rng.integers(-3, 6))
        nh = int(rng.integers(0, L + 1)) if rng.random() < 0.3 else None
        pat = None
        if rng.random() < 0.4:
            pat = "".join(rng.choice(["F", "S"], size=int(rng.integers(0, 90))))
        first = int(rng.integers(0, 70)) if rng.random() < 0.3 else 0
        step = int(rng.integers(0, 3))
        reuse = bool(rng.random() < 0.5)
        ours = binding.dsa_index_cache_mask(
            L, pattern=pat, freq=freq, offset=off,
            num_hidden_layers=-1 if nh is None else nh, first_layer=first,
            mtp_draft_step=step, mtp_reuse=reuse)
        ref = index_cache.skip_mask(L, pattern=pat, freq=freq, offset=off,
                                    num_hidden_layers=nh, first_layer=first,
                                    mtp_draft_step=step, mtp_reuse=reuse)
        assert ours == ref.tolist()


def _logits_call(**over):
    args = dict(q_fp8=None, q_scale=None, weights=None, k_cache=None,
                num_pages=4, block_table=None, bt_stride=4, qsl=None,
                positions=None, T=8, R=1, H=4, head_dim=128, page_size=64,
                logits=None, ld=256, stream=None)
    args.update(over)
    return binding.lib().dsa_indexer_logits(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), binding.DSA_ERR_UNSUPPORTED),
    (dict(page_size=32), binding.DSA_ERR_UNSUPPORTED),
    (dict(H=65), binding.DSA_ERR_UNSUPPORTED),
    (dict(H=0), binding.DSA_ERR_UNSUPPORTED),
    (dict(ld=100), binding.DSA_ERR_INVALID_ARG),
    (dict(ld=0), binding.DSA_ERR_INVALID_ARG),
    (dict(T=-1), binding.DSA_ERR_INVALID_ARG),
    (dict(R=0), binding.DSA_ERR_INVALID_ARG),
    (dict(bt_stride=0), binding.DSA_ERR_INVALID_ARG),
    (dict(num_pages=0), binding.DSA_ERR_INVALID_ARG),
    (dict(), binding.DSA_ERR_INVALID_ARG),          # null device pointers
])
def test_logits_rejects_bad_arguments(over, status):
    assert _logits_call(**over) == status
    assert binding.lib().dsa_last_error()


def test_logits_empty_batch_is_noop():
    assert _logits_call(T=0) == binding.DSA_OK


def test_topk_rejects_bad_arguments():
    L = binding.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.dsa_indexer_topk(fake, 100, fake, 4, 8, fake, 8, None, 0, None) \
        == binding.DSA_ERR_INVALID_ARG                        # ld % 256
    assert L.dsa_indexer_topk(fake, 256, fake, 4, 0, fake, 8, None, 0, None) \
        == binding.DSA_ERR_INVALID_ARG                        # k < 1
    assert L.dsa_indexer_topk(fake, 256, fake, 4, 8, fake, 4, None, 0, None) \
        == binding.DSA_ERR_INVALID_ARG                        # out_ld < k
    assert L.dsa_indexer_topk(None, 256, None, 4, 8, None, 8, None, 0, None) \
        == binding.DSA_ERR_INVALID_ARG                        # nulls
    assert L.dsa_indexer_topk(None, 256, None, 0, 8, None, 8, None, 0, None) \
        == binding.DSA_OK                                     # empty


def test_quantize_rejects_bad_arguments():
    L = binding.lib()
    assert L.dsa_quantize_q(None, 4, 4, 64, None, None, None) == \
        binding.DSA_ERR_UNSUPPORTED
    assert L.dsa_quantize_q(None, 4, 4, 128, None, None, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_q(None, 0, 4, 128, None, None, None) == binding.DSA_OK


def test_k_write_and_slot_mapping_reject_bad_arguments():
    L = binding.lib()
    assert L.dsa_indexer_k_write(None, 4, 64, None, None, 4, None) == \
        binding.DSA_ERR_UNSUPPORTED
    assert L.dsa_indexer_k_write(None, 4, 128, None, None, 4, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_indexer_k_write(None, -1, 128, None, None, 4, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_indexer_k_write(None, 0, 128, None, None, 4, None) == \
        binding.DSA_OK
    assert L.dsa_slot_mapping(None, 4, None, 1, None, 4, None, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_slot_mapping(None, 0, None, 1, None, 4, None, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_slot_mapping(None, 4, None, 1, None, 0, None, None) == \
        binding.DSA_OK


def test_compressed_slot_mapping_rejects_bad_arguments():
    L = binding.lib()
    P = ctypes.c_void_p(0x1000)
    f = L.dsa_compressed_slot_mapping
    assert f(P, 4, P, 1, P, 4, 0, 64, P, None, None) == \
        binding.DSA_ERR_INVALID_ARG                       # ratio < 1
    assert f(P, 4, P, 1, P, 4, 4, 0, P, None, None) == \
        binding.DSA_ERR_INVALID_ARG                       # block_size < 1
    assert f(P, 0, P, 1, P, 4, 4, 64, P, None, None) == \
        binding.DSA_ERR_INVALID_ARG                       # bt_stride < 1
    assert f(None, 4, P, 1, P, 4, 4, 64, P, None, None) == \
        binding.DSA_ERR_INVALID_ARG                       # null pointer
    assert f(None, 4, None, 1, None, 0, 4, 64, None, None, None) == \
        binding.DSA_OK                                    # T == 0


def test_handoff_rejects_bad_arguments():
    L = binding.lib()
    P = ctypes.c_void_p(0x1000)
    assert L.dsa_topk_to_slots(P, 4, 8, 4, P, 4, P, 1, P, None) == \
        binding.DSA_ERR_INVALID_ARG                       # topk_ld < k
    assert L.dsa_topk_to_slots(None, 4, 8, 8, P, 4, P, 1, P, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_topk_to_slots(None, 0, 8, 8, None, 4, None, 1, None,
                               None) == binding.DSA_OK
    assert L.dsa_topk_mask(P, 4, 8, 8, P, 100, None) == \
        binding.DSA_ERR_INVALID_ARG                       # ld % 256
    assert L.dsa_topk_mask(None, 4, 8, 8, None, 256, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_topk_mask(None, 0, 8, 8, None, 256, None) == binding.DSA_OK


def _fake_layers(n=3):
    arr = (binding.LayerInputs * n)()
    for i in range(n):
        arr[i] = binding.LayerInputs(0x1000, 0x1000, 0x1000, 4)
    return arr


def _run_call(**over):
    args = dict(pattern=None, freq=1, offset=2, first=0, L=3, nh=-1,
                step=0, reuse=0, layers=_fake_layers(),
                bt=ctypes.c_void_p(0x1000), bt_stride=4,
                qsl=ctypes.c_void_p(0x1000), pos=ctypes.c_void_p(0x1000),
                T=4, R=1, H=4, ld=256, k=8, rows=0,
                buf=ctypes.c_void_p(0x1000),
                buf_rows=4, snaps=None, skip=None,
                cb=binding.LAYER_CALLBACK(0), user=None,
                ws=ctypes.c_void_p(0x1000), ws_bytes=1 << 30, stream=None)
    args.update(over)
    return binding.lib().dsa_index_cache_run(*args.values())


def test_run_rejects_first_layer_s():
    assert _run_call(pattern=b"SFF") == binding.DSA_ERR_INVALID_ARG
    assert b"layer 0" in binding.lib().dsa_last_error()
    assert _run_call(freq=2, offset=0) == binding.DSA_ERR_INVALID_ARG


def test_run_mtp_reuse_pass_may_start_with_s():
    """An MTP draft pass at step > 0 with the reuse switch is all S and is
    accepted (no layer input is read); the same pass at step 0, or a trunk
    pass, with S first is still refused."""
    skip = (ctypes.c_uint8 * 2)()
    none = (binding.LayerInputs * 2)()
    assert _run_call(first=61, L=2, nh=61, step=1, reuse=1, layers=none,
                     skip=skip) == binding.DSA_OK
    assert list(skip) == [1, 1]
    assert _run_call(first=61, L=2, nh=61, step=0, reuse=1, layers=none) == \
        binding.DSA_ERR_INVALID_ARG                      # F with null inputs
    assert _run_call(pattern=b"SF", nh=61, step=1, reuse=1, L=2,
                     layers=_fake_layers(2)) == binding.DSA_ERR_INVALID_ARG
    assert _run_call(first=-1) == binding.DSA_ERR_INVALID_ARG
    assert _run_call(step=-1) == binding.DSA_ERR_INVALID_ARG


def test_run_rejects_negative_chunk_rows():
    assert _run_call(rows=-1) == binding.DSA_ERR_INVALID_ARG


def test_run_rejects_bad_arguments():
    assert _run_call(pattern=b"FXF") == binding.DSA_ERR_INVALID_ARG
    assert _run_call(freq=0) == binding.DSA_ERR_INVALID_ARG
    assert _run_call(ws_bytes=16) == binding.DSA_ERR_WORKSPACE
    assert _run_call(buf_rows=2) == binding.DSA_ERR_INVALID_ARG
    assert _run_call(k=0) == binding.DSA_ERR_INVALID_ARG
    assert _run_call(ld=300) == binding.DSA_ERR_INVALID_ARG
    # F layer with null inputs
    arr = (binding.LayerInputs * 3)()
    assert _run_call(layers=arr) == binding.DSA_ERR_INVALID_ARG
    assert b"layer 0" in binding.lib().dsa_last_error()


def test_run_with_no_rows_only_reports_mask():
    skip = (ctypes.c_uint8 * 5)()
    assert _run_call(L=5, freq=2, offset=1, T=0, layers=_fake_layers(5),
                     skip=skip, ws=None, ws_bytes=0) == binding.DSA_OK
    assert list(skip) == [0, 1, 0, 1, 0]


def test_workspace_sizes():
    assert binding.dsa_run_workspace_size(64, 64, 64, 8192, 2048) >= \
        64 * 64 * 128 + 64 * 64 * 4 + 64 * 8192 * 4
    assert binding.dsa_run_workspace_size(0, 64, 64, 8192, 2048) == 0
    # chunked: the logits of rows_per_chunk rows instead of all T
    full = binding.dsa_run_workspace_size(4096, 1, 64, 40960, 2048)
    ch = binding.dsa_run_workspace_size(4096, 1, 64, 40960, 2048, 512)
    assert ch == binding.dsa_forward_chunked_workspace_size(4096, 1, 64,
                                                            40960, 2048, 512)
    assert full - ch >= (4096 - 512) * 40960 * 4 - (1 << 20)
    assert binding.dsa_run_workspace_size(4096, 1, 64, 40960, 2048, 4096) == \
        full


def test_mfma_rate_probe_rejects_bad_arguments():
    L = binding.lib()
    flops = ctypes.c_double(0.0)
    for iters in (0, -5, (1 << 24) + 1):
        assert L.dsa_fp8_mfma_rate_probe(iters, ctypes.byref(flops),
                                         None) == binding.DSA_ERR_INVALID_ARG
    assert L.dsa_fp8_mfma_rate_probe(16, None, None) == \
        binding.DSA_ERR_INVALID_ARG


def test_page_read_probe_rejects_bad_arguments():
    L = binding.lib()
    dummy = ctypes.c_void_p(0x1000)
    assert L.dsa_page_read_probe(dummy, 16, dummy, -1, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_page_read_probe(dummy, 0, dummy, 4, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_page_read_probe(None, 16, dummy, 4, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_page_read_probe(dummy, 16, None, 4, None) == \
        binding.DSA_ERR_INVALID_ARG
    assert L.dsa_page_read_probe(dummy, 16, dummy, (1 << 31) + 1, None) == \
        binding.DSA_ERR_UNSUPPORTED
    assert L.dsa_page_read_probe(None, 16, None, 0, None) == binding.DSA_OK


def test_set_option_roundtrip():
    prev = binding.dsa_set_option("logits_kernel", 2)
    assert binding.dsa_set_option("logits_kernel", prev) == 2
    with pytest.raises(binding.DsaError):
        binding.dsa_set_option("no_such_knob", 1)


def test_logits_budget_and_chunk_rows_match_oracle():
    from oracle import chunking
    import numpy as np
    rng = np.random.default_rng(12)
    for total in (0, 1, 10**9, 288 * 10**9, 2**40 + 7):
        for mfs in (None, 0.0, 0.5, 0.85, 1.0, 1.5):
            for free in (1.0, 0.25):
                assert binding.dsa_logits_budget_bytes(total, mfs, free) == \
                    chunking.budget_bytes(total, mfs, free), (total, mfs, free)
    for _ in range(2000):
        T = int(rng.integers(0, 70000))
        ld = 256 * int(rng.integers(1, 5000))
        budget = int(rng.integers(1, 1 << 36))
        assert binding.dsa_logits_chunk_rows(T, ld, budget) == \
            chunking.chunk_rows(T, ld, budget), (T, ld, budget)


def test_forward_chunked_rejects_bad_arguments():
    L = binding.lib()
    P = ctypes.c_void_p(0x1000)
    base = dict(q=P, w=P, kc=P, npg=4, bt=P, bts=4, qsl=P, pos=P, T=4, R=1,
                H=16, D=128, ps=64, ld=256, k=8, out=P, out_ld=8, rows=2,
                ws=P, ws_bytes=1 << 30, stream=None)

    def call(**over):
        a = dict(base)
        a.update(over)
        return L.dsa_indexer_forward_chunked(*a.values())
    assert call(rows=0) == binding.DSA_ERR_INVALID_ARG
    assert call(k=0) == binding.DSA_ERR_INVALID_ARG
    assert call(out_ld=4) == binding.DSA_ERR_INVALID_ARG
    assert call(ld=300) == binding.DSA_ERR_INVALID_ARG
    assert call(D=64) == binding.DSA_ERR_UNSUPPORTED
    assert call(ws_bytes=16) == binding.DSA_ERR_WORKSPACE
    assert call(out=None) == binding.DSA_ERR_INVALID_ARG
    assert call(T=0, ws=None, ws_bytes=0) == binding.DSA_OK
    need = binding.dsa_forward_chunked_workspace_size(4, 1, 16, 256, 8, 2)
    assert need >= 4 * 16 * 132 + 2 * 256 * 4 + 8
    assert binding.dsa_forward_chunked_workspace_size(4, 1, 16, 256, 8, 0) == 0


def test_missing_library_raises(monkeypatch):
    """No CPU fallback: without the built library every entry point raises
    before doing anything."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libdsa_indexer.so")
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        binding.dsa_index_cache_mask(4)
    with pytest.raises(RuntimeError, match="missing"):
        binding.dsa_logits_chunk_rows(8, 256, 1 << 20)


def _imports(path):
    import ast
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0:
            yield node.module or ""


def test_product_and_oracle_share_no_code():
    """The product path (binding, build, synthetic inputs) and the oracle
    import nothing of each other."""
    import os
    pkg = os.path.dirname(binding.__file__)
    root = os.path.dirname(pkg)
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            for m in _imports(os.path.join(pkg, name)):
                assert m.split(".")[0] != "oracle", (name, m)
    for name in os.listdir(os.path.join(root, "oracle")):
        if name.endswith(".py"):
            for m in _imports(os.path.join(root, "oracle", name)):
                assert m.split(".")[0] != "dsa_lightning_indexer_amd", (name, m)


def test_fp8_code_check_rejects_null_counts():
    L = binding.lib()
    assert L.dsa_fp8_code_check(None, None) == binding.DSA_ERR_INVALID_ARG
