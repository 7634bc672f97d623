"""Python binding of libdsa_indexer.so (ctypes).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Tensors are torch tensors on the GPU (PyTorch provides device
memory and the stream); each function passes ``data_ptr()``s, sizes and
``torch.cuda.current_stream().cuda_stream`` to the C entry point of the same
name (declared in include/dsa_indexer.h) and raises ``DsaError`` on a
non-zero status.  There is no fallback: if the library is missing, the first
call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libdsa_indexer.so")

DSA_OK = 0
DSA_ERR_INVALID_ARG = -1
DSA_ERR_UNSUPPORTED = -2
DSA_ERR_WORKSPACE = -3
DSA_ERR_HIP = -4

HEAD_DIM = 128
PAGE_TOKENS = 64
PAGE_BYTES = 8448
LOGITS_ROW_ALIGN = 256


class DsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"dsa status {status}: {message}")
        self.status = status


class LayerInputs(ctypes.Structure):
    _fields_ = [("q_bf16", ctypes.c_void_p), ("weights", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("num_pages", ctypes.c_int64)]


LAYER_CALLBACK = ctypes.CFUNCTYPE(None, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p)

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_S = ctypes.c_size_t
_SIGNATURES = {
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_version": (_I, []),
    "dsa_quantize_q": (_I, [_P, _L, _I, _I, _P, _P, _P]),
    "dsa_indexer_logits": (_I, [_P, _P, _P, _P, _L, _P, _L, _P, _P, _L, _I,
                                _I, _I, _I, _P, _L, _P]),
    "dsa_indexer_topk": (_I, [_P, _L, _P, _L, _I, _P, _L, _P, _S, _P]),
    "dsa_topk_workspace_size": (_S, [_L, _L, _I]),
    "dsa_logits_schedule_size": (_S, [_L, _L]),
    "dsa_logits_schedule": (_I, [_P, _L, _P, _P, _L, _I, _L, _P, _S, _P]),
    "dsa_indexer_logits_scheduled": (_I, [_P, _P, _P, _P, _L, _P, _L, _P, _P,
                                          _L, _I, _I, _I, _I, _P, _L, _P,
                                          _P]),
    "dsa_indexer_forward": (_I, [_P, _P, _P, _L, _P, _L, _P, _P, _L, _I, _I,
                                 _I, _I, _P, _L, _I, _P, _L, _P, _S, _P]),
    "dsa_forward_workspace_size": (_S, [_L, _I, _L, _I]),
    "dsa_indexer_forward_noalloc": (_I, [_P, _P, _P, _L, _P, _L, _P, _P, _L,
                                         _I, _I, _I, _I, _P, _L, _I, _P, _L,
                                         _P]),
    "dsa_logits_budget_bytes": (_S, [_S, ctypes.c_double, ctypes.c_double]),
    "dsa_logits_chunk_rows": (_L, [_L, _L, _S]),
    "dsa_indexer_forward_chunked": (_I, [_P, _P, _P, _L, _P, _L, _P, _P, _L,
                                         _I, _I, _I, _I, _L, _I, _P, _L, _L,
                                         _P, _S, _P]),
    "dsa_forward_chunked_workspace_size": (_S, [_L, _I, _I, _L, _I, _L]),
    "dsa_indexer_forward_fused": (_I, [_P, _P, _P, _L, _P, _L, _P, _P, _L,
                                       _I, _I, _I, _I, _L, _I, _P, _L, _P,
                                       _S, _P]),
    "dsa_forward_fused_workspace_size": (_S, [_L, _I, _I, _L, _I]),
    "dsa_index_cache_mask": (_I, [ctypes.c_char_p, _I, _I, _I, _I, _I, _I,
                                  _I, _P]),
    "dsa_index_cache_run": (_I, [ctypes.c_char_p, _I, _I, _I, _I, _I, _I, _I,
                                 _P, _P, _L, _P, _P, _L, _I, _I, _L, _I, _L,
                                 _P, _L, _P, _P, LAYER_CALLBACK, _P, _P, _S,
                                 _P]),
    "dsa_run_workspace_size": (_S, [_L, _I, _I, _L, _I, _L]),
    "dsa_slot_mapping": (_I, [_P, _L, _P, _I, _P, _L, _P, _P]),
    "dsa_compressed_slot_mapping": (_I, [_P, _L, _P, _I, _P, _L, _I, _I, _P,
                                         _P, _P]),
    "dsa_indexer_k_write": (_I, [_P, _L, _I, _P, _P, _L, _P]),
    "dsa_topk_to_slots": (_I, [_P, _L, _I, _L, _P, _L, _P, _I, _P, _P]),
    "dsa_topk_mask": (_I, [_P, _L, _I, _L, _P, _L, _P]),
    "dsa_device_error_flags": (_I, [_I]),
    "dsa_fp8_mfma_rate_probe": (_I, [_I, ctypes.POINTER(ctypes.c_double),
                                     _P]),
    "dsa_page_read_probe": (_I, [_P, _L, _P, _L, _P]),
    "dsa_fp8_code_check": (_I, [_P, _P]),
    "dsa_set_option": (_I, [ctypes.c_char_p, _I]),
}


def lib():
    """The loaded library (loads it on first use; raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m dsa_lightning_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc < 0:
        msg = lib().dsa_last_error()
        raise DsaError(rc, msg.decode() if msg else "")
    return rc


def _dev_ptr(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t, shape, name):
    """Raise ValueError unless tensor ``t`` has ``shape`` (None = any
    extent on that axis)."""
    if t is None:
        return
    got = tuple(t.shape)
    if len(got) != len(shape) or any(
            w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")


def _rows_at_least(t, rows, name, cols=None):
    """Raise ValueError unless 2-D ``t`` has >= ``rows`` rows (and, when
    given, >= ``cols`` columns)."""
    if t.dim() != 2 or t.shape[0] < rows or (cols is not None and
                                             t.shape[1] < cols):
        raise ValueError(f"{name} must be 2-D with at least {rows} rows"
                         + (f" and {cols} columns" if cols is not None else "")
                         + f", got {tuple(t.shape)}")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def dsa_quantize_q(q_bf16, q_fp8=None, q_scale=None, stream=None):
    """bf16 [T, H, 128] -> (uint8 codes [T, H, 128], fp32 scales [T, H])."""
    T, H, D = q_bf16.shape
    dev = q_bf16.device
    if q_fp8 is None:
        q_fp8 = torch.empty((T, H, D), dtype=torch.uint8, device=dev)
    if q_scale is None:
        q_scale = torch.empty((T, H), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_quantize_q(
            _dev_ptr(q_bf16, torch.bfloat16, "q_bf16"), T, H, D,
            _dev_ptr(q_fp8, torch.uint8, "q_fp8"),
            _dev_ptr(q_scale, torch.float32, "q_scale"), _stream(stream, dev)))
    return q_fp8, q_scale


def dsa_indexer_logits(q_fp8, q_scale, weights, k_cache, block_table,
                       query_start_loc, positions, ld, logits=None,
                       stream=None):
    """Causal indexer logits, fp32 [T, ld]."""
    T, H, D = q_fp8.shape
    R = block_table.shape[0]
    dev = q_fp8.device
    if logits is None:
        logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(q_scale, (T, H), "q_scale")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(logits, T, "logits")
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_logits(
            _dev_ptr(q_fp8, torch.uint8, "q_fp8"),
            _dev_ptr(q_scale, torch.float32, "q_scale"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, _dev_ptr(logits, torch.float32, "logits"),
            logits.shape[1], _stream(stream, dev)))
    return logits


def dsa_logits_schedule_size(T, ld):
    return lib().dsa_logits_schedule_size(T, ld)


def dsa_logits_schedule(block_table, query_start_loc, positions, ld,
                        schedule=None, stream=None):
    """Decode page schedule (int32 device buffer) of a batch for
    dsa_indexer_logits_scheduled; None when the batch takes none."""
    T = positions.shape[0]
    R = block_table.shape[0]
    dev = positions.device
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    need = dsa_logits_schedule_size(T, ld)
    if need == 0:
        return None
    if schedule is None:
        schedule = torch.empty((need // 4,), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_logits_schedule(
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, ld,
            _dev_ptr(schedule, torch.int32, "schedule"),
            schedule.numel() * 4, _stream(stream, dev)))
    return schedule


def dsa_indexer_logits_scheduled(q_fp8, q_scale, weights, k_cache,
                                 block_table, query_start_loc, positions, ld,
                                 schedule, logits=None, stream=None):
    """dsa_indexer_logits with a schedule from dsa_logits_schedule (same
    results)."""
    T, H, D = q_fp8.shape
    R = block_table.shape[0]
    dev = q_fp8.device
    if logits is None:
        logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(q_scale, (T, H), "q_scale")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(logits, T, "logits")
    if schedule is not None and \
            schedule.numel() * 4 < dsa_logits_schedule_size(T, ld):
        raise ValueError("schedule smaller than dsa_logits_schedule_size")
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_logits_scheduled(
            _dev_ptr(q_fp8, torch.uint8, "q_fp8"),
            _dev_ptr(q_scale, torch.float32, "q_scale"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, _dev_ptr(logits, torch.float32, "logits"),
            logits.shape[1], _dev_ptr(schedule, torch.int32, "schedule"),
            _stream(stream, dev)))
    return logits


def dsa_topk_workspace_size(T, ld, k):
    return lib().dsa_topk_workspace_size(T, ld, k)


def dsa_indexer_topk(logits, positions, k, out=None, workspace=None,
                     stream=None):
    """Per-row causal top-k, int32 [T, k] (ascending positions, -1 padded)."""
    T, ld = logits.shape
    dev = logits.device
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=dev)
    _shape(positions, (T,), "positions")
    _rows_at_least(out, T, "out", k)
    need = dsa_topk_workspace_size(T, ld, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = _dev_ptr(workspace, torch.uint8, "workspace") if need > 0 else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_topk(
            _dev_ptr(logits, torch.float32, "logits"), ld,
            _dev_ptr(positions, torch.int32, "positions"), T, k,
            _dev_ptr(out, torch.int32, "out"), out.shape[1], ws_ptr, ws_bytes,
            _stream(stream, dev)))
    return out


def dsa_forward_workspace_size(T, H, ld, k):
    return lib().dsa_forward_workspace_size(T, H, ld, k)


def dsa_indexer_forward(q_bf16, weights, k_cache, block_table,
                        query_start_loc, positions, ld, k, logits=None,
                        out=None, workspace=None, stream=None):
    """One layer's hot path: q quantisation, logits and top-k.  Returns
    (logits fp32 [T, ld], top-k int32 [T, k])."""
    T, H, D = q_bf16.shape
    R = block_table.shape[0]
    dev = q_bf16.device
    if logits is None:
        logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=dev)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(logits, T, "logits")
    _rows_at_least(out, T, "out", k)
    need = dsa_forward_workspace_size(T, H, logits.shape[1], k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_forward(
            _dev_ptr(q_bf16, torch.bfloat16, "q_bf16"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, _dev_ptr(logits, torch.float32, "logits"),
            logits.shape[1], k, _dev_ptr(out, torch.int32, "out"),
            out.shape[1], _dev_ptr(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream(stream, dev)))
    return logits, out


NOALLOC_SCRATCH_BYTES = 32 << 20


def dsa_indexer_forward_noalloc(q_bf16, weights, k_cache, block_table,
                                query_start_loc, positions, logits, out,
                                k=None, stream=None):
    """dsa_indexer_forward without a workspace: the library's own fixed
    scratch array is used (no device allocation in the call).  ``logits``
    (fp32 [>= T, ld]) and ``out`` (int32 [>= T, >= k]) are the caller's;
    k defaults to out's width.  Returns (logits, out)."""
    T, H, D = q_bf16.shape
    R = block_table.shape[0]
    dev = q_bf16.device
    k = out.shape[1] if k is None else int(k)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(logits, T, "logits")
    _rows_at_least(out, T, "out", k)
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_forward_noalloc(
            _dev_ptr(q_bf16, torch.bfloat16, "q_bf16"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, _dev_ptr(logits, torch.float32, "logits"),
            logits.shape[1], k, _dev_ptr(out, torch.int32, "out"),
            out.shape[1], _stream(stream, dev)))
    return logits, out


def dsa_logits_budget_bytes(total_mem, mem_fraction_static=None,
                            free_mem_fraction=1.0):
    return lib().dsa_logits_budget_bytes(
        int(total_mem),
        -1.0 if mem_fraction_static is None else float(mem_fraction_static),
        float(free_mem_fraction))


def dsa_logits_chunk_rows(T, ld, budget_bytes):
    return lib().dsa_logits_chunk_rows(T, ld, int(budget_bytes))


def dsa_forward_chunked_workspace_size(T, R, H, ld, k, rows_per_chunk):
    return lib().dsa_forward_chunked_workspace_size(T, R, H, ld, k,
                                                    rows_per_chunk)


def dsa_indexer_forward_chunked(q_bf16, weights, k_cache, block_table,
                                query_start_loc, positions, ld, k,
                                rows_per_chunk=None, budget_bytes=None,
                                out=None, workspace=None, stream=None):
    """The forward pass over row chunks that share one logits buffer of
    ``rows_per_chunk`` rows (default: the rows ``budget_bytes`` allows, and
    the budget defaults to 30 % of the device's memory).  Returns the top-k
    int32 [T, k]."""
    T, H, D = q_bf16.shape
    R = block_table.shape[0]
    dev = q_bf16.device
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=dev)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(out, T, "out", k)
    if rows_per_chunk is None:
        if budget_bytes is None:
            total = torch.cuda.get_device_properties(dev).total_memory
            budget_bytes = dsa_logits_budget_bytes(total)
        rows_per_chunk = max(1, dsa_logits_chunk_rows(T, ld, budget_bytes))
    need = dsa_forward_chunked_workspace_size(T, R, H, ld, k, rows_per_chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_forward_chunked(
            _dev_ptr(q_bf16, torch.bfloat16, "q_bf16"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, ld, k, _dev_ptr(out, torch.int32, "out"),
            out.shape[1], rows_per_chunk,
            _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
            _stream(stream, dev)))
    return out


def dsa_forward_fused_workspace_size(T, R, H, ld, k):
    return lib().dsa_forward_fused_workspace_size(T, R, H, ld, k)


def dsa_indexer_forward_fused(q_bf16, weights, k_cache, block_table,
                              query_start_loc, positions, ld, k, out=None,
                              workspace=None, stream=None):
    """The forward pass without a logits buffer (scoring with candidate
    filtering, then the top-k of the candidates).  Returns the top-k int32
    [T, k]."""
    T, H, D = q_bf16.shape
    R = block_table.shape[0]
    dev = q_bf16.device
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=dev)
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    _shape(weights, (T, H), "weights")
    _shape(positions, (T,), "positions")
    _rows_at_least(out, T, "out", k)
    need = dsa_forward_fused_workspace_size(T, R, H, ld, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_forward_fused(
            _dev_ptr(q_bf16, torch.bfloat16, "q_bf16"),
            _dev_ptr(weights, torch.float32, "weights"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, D,
            PAGE_TOKENS, ld, k, _dev_ptr(out, torch.int32, "out"),
            out.shape[1], _dev_ptr(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream(stream, dev)))
    return out


def dsa_index_cache_mask(num_layers, pattern=None, freq=1, offset=2,
                         num_hidden_layers=-1, first_layer=0,
                         mtp_draft_step=0, mtp_reuse=False):
    """IndexCache F/S mask (host) of layer ids first_layer ..
    first_layer + num_layers - 1: list of bools, True = S (reuse)."""
    buf = (ctypes.c_uint8 * max(num_layers, 1))()
    pat = pattern.encode() if pattern is not None else None
    _check(lib().dsa_index_cache_mask(pat, freq, offset, first_layer,
                                      num_layers, num_hidden_layers,
                                      mtp_draft_step, int(bool(mtp_reuse)),
                                      buf))
    return [bool(buf[i]) for i in range(num_layers)]


def dsa_run_workspace_size(T, R, H, ld, k, rows_per_chunk=0):
    return lib().dsa_run_workspace_size(T, R, H, ld, k, rows_per_chunk)


def dsa_index_cache_run(layers, block_table, query_start_loc, positions, ld,
                        k, topk_buffer, pattern=None, freq=1, offset=2,
                        num_hidden_layers=-1, H=None, snapshots=False,
                        callback=None, workspace=None, stream=None,
                        first_layer=0, mtp_draft_step=0, mtp_reuse=False,
                        rows_per_chunk=0):
    """One forward pass over ``len(layers)`` DSA layers (ids first_layer ..).

    ``layers[l]`` is a dict with ``q_bf16`` (bf16 [T, H, 128]), ``weights``
    (fp32 [T, H]) and ``k_cache`` (uint8 [pages, 8448]) for F layers, or None
    (allowed for S layers).  Returns (is_skip list, snapshots tensor
    [L, T, k] or None).
    """
    L = len(layers)
    T = positions.numel()
    R = block_table.shape[0]
    dev = topk_buffer.device
    if topk_buffer.dim() != 2 or topk_buffer.shape[1] != k:
        raise ValueError("topk_buffer must be int32 [buffer_rows, k]")
    if H is None:
        H = next((l["q_bf16"].shape[1] for l in layers if l is not None), 1)
    arr = (LayerInputs * max(L, 1))()
    for i, lay in enumerate(layers):
        if lay is not None:
            _shape(lay["q_bf16"], (T, H, HEAD_DIM), f"layers[{i}].q_bf16")
            _shape(lay["weights"], (T, H), f"layers[{i}].weights")
            if lay["k_cache"].dim() != 2 or \
                    lay["k_cache"].shape[1] != PAGE_BYTES:
                raise ValueError(f"layers[{i}].k_cache must be uint8 "
                                 "[num_pages, 8448]")
        if lay is None:
            arr[i] = LayerInputs(None, None, None, 0)
        else:
            arr[i] = LayerInputs(
                _dev_ptr(lay["q_bf16"], torch.bfloat16, "q_bf16"),
                _dev_ptr(lay["weights"], torch.float32, "weights"),
                _dev_ptr(lay["k_cache"], torch.uint8, "k_cache"),
                lay["k_cache"].shape[0])
    snaps = torch.empty((L, T, k), dtype=torch.int32, device=dev) \
        if snapshots else None
    need = dsa_run_workspace_size(T, R, H, ld, k, rows_per_chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    skip = (ctypes.c_uint8 * max(L, 1))()
    cb = LAYER_CALLBACK(0) if callback is None else LAYER_CALLBACK(
        lambda layer, full, buf, user: callback(layer, bool(full)))
    pat = pattern.encode() if pattern is not None else None
    with torch.cuda.device(dev):
        _check(lib().dsa_index_cache_run(
            pat, freq, offset, first_layer, L, num_hidden_layers,
            mtp_draft_step, int(bool(mtp_reuse)), arr,
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"),
            _dev_ptr(positions, torch.int32, "positions"), T, R, H, ld, k,
            rows_per_chunk, _dev_ptr(topk_buffer, torch.int32, "topk_buffer"),
            topk_buffer.shape[0],
            _dev_ptr(snaps, torch.int32, "snapshots") if snaps is not None
            else None, skip, cb, None,
            _dev_ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
            _stream(stream, dev)))
    return [bool(skip[i]) for i in range(L)], snaps


def dsa_slot_mapping(block_table, query_start_loc, positions, slots=None,
                     stream=None):
    """int64 [T] physical slot of every row's token (-1: no page)."""
    T = positions.shape[0]
    R = block_table.shape[0]
    dev = positions.device
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    if slots is None:
        slots = torch.empty((T,), dtype=torch.int64, device=dev)
    _shape(slots, (T,), "slots")
    with torch.cuda.device(dev):
        _check(lib().dsa_slot_mapping(
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"), R,
            _dev_ptr(positions, torch.int32, "positions"), T,
            _dev_ptr(slots, torch.int64, "slots"), _stream(stream, dev)))
    return slots


def dsa_compressed_slot_mapping(block_table, query_start_loc, positions,
                                compress_ratio, block_size, slots=None,
                                positions_c=None, want_positions_c=True,
                                stream=None):
    """(int64 [T] compressed-cache slots, -1 off the ratio boundary;
    int32 [T] compressed positions or None)."""
    T = positions.shape[0]
    R = block_table.shape[0]
    dev = positions.device
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    if slots is None:
        slots = torch.empty((T,), dtype=torch.int64, device=dev)
    if positions_c is None and want_positions_c:
        positions_c = torch.empty((T,), dtype=torch.int32, device=dev)
    _shape(slots, (T,), "slots")
    _shape(positions_c, (T,), "positions_c")
    with torch.cuda.device(dev):
        _check(lib().dsa_compressed_slot_mapping(
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"), R,
            _dev_ptr(positions, torch.int32, "positions"), T,
            int(compress_ratio), int(block_size),
            _dev_ptr(slots, torch.int64, "slots"),
            _dev_ptr(positions_c, torch.int32, "positions_c"),
            _stream(stream, dev)))
    return slots, positions_c


def dsa_indexer_k_write(k_bf16, slot_mapping, k_cache, stream=None):
    """Quantise bf16 keys [N, 128] and store them at their slots of
    k_cache (uint8 [num_pages, 8448], modified in place)."""
    N, D = k_bf16.shape
    dev = k_bf16.device
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if slot_mapping.numel() != N:
        raise ValueError("slot_mapping must have one entry per key")
    with torch.cuda.device(dev):
        _check(lib().dsa_indexer_k_write(
            _dev_ptr(k_bf16, torch.bfloat16, "k_bf16"), N, D,
            _dev_ptr(slot_mapping, torch.int64, "slot_mapping"),
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _stream(stream, dev)))
    return k_cache


def dsa_topk_to_slots(topk, block_table, query_start_loc, slots=None,
                      stream=None, k=None):
    """int64 [T, k] physical slot of every top-k entry (-1 stays -1); the
    first k (default: all) entries of each topk row are used."""
    T, width = topk.shape
    k = width if k is None else int(k)
    R = block_table.shape[0]
    dev = topk.device
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must have R + 1 entries")
    if slots is None:
        slots = torch.empty((T, k), dtype=torch.int64, device=dev)
    _shape(slots, (T, k), "slots")
    with torch.cuda.device(dev):
        _check(lib().dsa_topk_to_slots(
            _dev_ptr(topk, torch.int32, "topk"), T, k, width,
            _dev_ptr(block_table, torch.int32, "block_table"),
            block_table.shape[1],
            _dev_ptr(query_start_loc, torch.int32, "query_start_loc"), R,
            _dev_ptr(slots, torch.int64, "slots"), _stream(stream, dev)))
    return slots


def dsa_topk_mask(topk, ld, mask=None, stream=None, k=None):
    """fp32 [T, ld]: 0 at the selected columns, -inf elsewhere; the first k
    (default: all) entries of each topk row are used."""
    T, width = topk.shape
    k = width if k is None else int(k)
    dev = topk.device
    if mask is None:
        mask = torch.empty((T, ld), dtype=torch.float32, device=dev)
    _shape(mask, (T, ld), "mask")
    with torch.cuda.device(dev):
        _check(lib().dsa_topk_mask(
            _dev_ptr(topk, torch.int32, "topk"), T, k, width,
            _dev_ptr(mask, torch.float32, "mask"), ld, _stream(stream, dev)))
    return mask


def dsa_device_error_flags(reset=True):
    return _check(lib().dsa_device_error_flags(1 if reset else 0))


def dsa_fp8_mfma_rate_probe(iters, stream=None, device=None):
    """Enqueue one pure FP8 MFMA loop launch on the current (or given)
    device (measurement helper); returns the FP8 operations it performs
    (time it with events on the stream)."""
    dev = torch.device("cuda", torch.cuda.current_device()) \
        if device is None else torch.device(device)
    flops = ctypes.c_double(0.0)
    with torch.cuda.device(dev):
        _check(lib().dsa_fp8_mfma_rate_probe(int(iters), ctypes.byref(flops),
                                             _stream(stream, dev)))
    return flops.value


def dsa_page_read_probe(k_cache, page_ids, stream=None):
    """Enqueue one bare read of the K pages page_ids (int32 [n]) of k_cache
    (uint8 [num_pages, 8448]) on the current stream (measurement helper;
    time it with events on the stream)."""
    if k_cache.dim() != 2 or k_cache.shape[1] != PAGE_BYTES:
        raise ValueError("k_cache must be uint8 [num_pages, 8448]")
    if page_ids.dim() != 1:
        raise ValueError("page_ids must be int32 [n]")
    dev = k_cache.device
    with torch.cuda.device(dev):
        _check(lib().dsa_page_read_probe(
            _dev_ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
            _dev_ptr(page_ids, torch.int32, "page_ids"), page_ids.numel(),
            _stream(stream, dev)))


def dsa_fp8_code_check(device=None, stream=None):
    """Run the exhaustive FP8 code check of the q quantisation's fast path
    on ``device``; returns the three mismatch counts (hardware conversion vs
    integer encoder, corrected quotient vs IEEE quotient, codes of the two
    quotients).  Synchronises."""
    dev = torch.device("cuda", 0) if device is None else torch.device(device)
    counts = torch.zeros(3, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        _check(lib().dsa_fp8_code_check(counts.data_ptr(),
                                        _stream(stream, dev)))
        torch.cuda.synchronize(dev)
    return [int(x) for x in counts.cpu().tolist()]


def dsa_set_option(key, value):
    return _check(lib().dsa_set_option(key.encode(), int(value)))
