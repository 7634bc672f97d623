"""The Python binding checks every tensor's shape against the sizes it
passes to the C ABI (rows T, heads H, logits columns ld, k) and raises
ValueError before the call: a mismatch would otherwise become an
out-of-bounds device access.  CPU tensors suffice, since the shape checks
come before the device-pointer checks."""

import pytest
import torch

from dsa_lightning_indexer_amd import binding

T, H, ld, k = 4, 8, 256, 16


def _t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _geo(R=4):
    return (_t(R, 4, dtype=torch.int32),                 # block_table
            torch.arange(R + 1, dtype=torch.int32))      # query_start_loc


def test_logits_shapes():
    bt, qsl = _geo()
    q8 = _t(T, H, 128, dtype=torch.uint8)
    kc = _t(10, 8448, dtype=torch.uint8)
    pos = _t(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="q_scale"):
        binding.dsa_indexer_logits(q8, _t(T, H + 1), _t(T, H), kc, bt, qsl,
                                   pos, ld)
    with pytest.raises(ValueError, match="weights"):
        binding.dsa_indexer_logits(q8, _t(T, H), _t(T - 1, H), kc, bt, qsl,
                                   pos, ld)
    with pytest.raises(ValueError, match="positions"):
        binding.dsa_indexer_logits(q8, _t(T, H), _t(T, H), kc, bt, qsl,
                                   _t(T + 1, dtype=torch.int32), ld)
    with pytest.raises(ValueError, match="logits"):
        binding.dsa_indexer_logits(q8, _t(T, H), _t(T, H), kc, bt, qsl, pos,
                                   ld, logits=_t(T - 1, ld))


def test_topk_shapes():
    lg = _t(T, ld)
    with pytest.raises(ValueError, match="positions"):
        binding.dsa_indexer_topk(lg, _t(T - 1, dtype=torch.int32), k)
    with pytest.raises(ValueError, match="out"):
        binding.dsa_indexer_topk(lg, _t(T, dtype=torch.int32), k,
                                 out=_t(T, k - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        binding.dsa_indexer_topk(lg, _t(T, dtype=torch.int32), k,
                                 out=_t(T - 1, k, dtype=torch.int32))


def test_forward_shapes():
    bt, qsl = _geo()
    q = _t(T, H, 128, dtype=torch.bfloat16)
    kc = _t(10, 8448, dtype=torch.uint8)
    pos = _t(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="weights"):
        binding.dsa_indexer_forward(q, _t(T, H - 1), kc, bt, qsl, pos, ld, k)
    with pytest.raises(ValueError, match="out"):
        binding.dsa_indexer_forward(q, _t(T, H), kc, bt, qsl, pos, ld, k,
                                    out=_t(T, k - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="positions"):
        binding.dsa_indexer_forward_chunked(q, _t(T, H), kc, bt, qsl,
                                            _t(2, dtype=torch.int32), ld, k,
                                            rows_per_chunk=1)


def test_hand_off_and_slot_shapes():
    bt, qsl = _geo()
    tk = _t(T, k, dtype=torch.int32)
    with pytest.raises(ValueError, match="mask"):
        binding.dsa_topk_mask(tk, ld, mask=_t(T, ld + 256))
    with pytest.raises(ValueError, match="slots"):
        binding.dsa_topk_to_slots(tk, bt, qsl,
                                  slots=_t(T, k + 1, dtype=torch.int64))
    with pytest.raises(ValueError, match="slots"):
        binding.dsa_slot_mapping(bt, qsl, _t(T, dtype=torch.int32),
                                 slots=_t(T - 1, dtype=torch.int64))


def test_run_layer_shapes():
    bt, qsl = _geo()
    lay = {"q_bf16": _t(T, H, 128, dtype=torch.bfloat16),
           "weights": _t(T, H + 2),
           "k_cache": _t(10, 8448, dtype=torch.uint8)}
    with pytest.raises(ValueError, match="weights"):
        binding.dsa_index_cache_run([lay], bt, qsl, _t(T, dtype=torch.int32),
                                    ld, k, _t(T, k, dtype=torch.int32))
