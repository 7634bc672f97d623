"""Pins for the oracle's e4m3fn codec (CPU only).

The codec is pinned against the format's closed form at spot values and
against torch's float8_e4m3fn conversions (a library routine, used here only
as a reference, never by the oracle itself).
"""

import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_spot_values():
    assert fp8.decode(np.uint8(0x7E)) == 448.0
    assert fp8.decode(np.uint8(0xFE)) == -448.0
    assert fp8.decode(np.uint8(0x08)) == 2.0 ** -6       # smallest normal
    assert fp8.decode(np.uint8(0x01)) == 2.0 ** -9       # smallest subnormal
    assert fp8.decode(np.uint8(0x07)) == 7 * 2.0 ** -9   # largest subnormal
    assert fp8.decode(np.uint8(0x38)) == 1.0             # E=7, M=0
    assert fp8.decode(np.uint8(0x3C)) == 1.5
    assert np.isnan(fp8.decode(np.uint8(0x7F)))
    assert np.isnan(fp8.decode(np.uint8(0xFF)))
    z = fp8.decode(np.uint8(0x80))
    assert z == 0.0 and np.signbit(z)


def test_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float() \
        .double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2


def test_positive_values_monotonic_and_count():
    v = fp8.positive_code_values()
    assert v.shape == (127,)
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0


def test_encode_exact_codes_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                     dtype=np.uint8)
    vals = fp8.decode(codes).astype(np.float32)
    assert np.array_equal(fp8.encode(vals), codes)


def _torch_encode(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_random_vs_torch():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(20000) * 100,
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** -7,      # subnormal range
        rng.standard_normal(5000) * 2.0 ** -11,      # rounds toward zero
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(fp8.encode(x), _torch_encode(x))


def test_encode_midpoints_ties_to_even():
    v = fp8.positive_code_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    # every midpoint between adjacent finite codes is exact in float32
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)
    ours = fp8.encode(mids)
    assert np.all(ours % 2 == 0)                      # even mantissa wins
    assert np.array_equal(ours, _torch_encode(mids))
    assert np.array_equal(fp8.encode(-mids), _torch_encode(-mids))
    # one float32 ulp either side of each midpoint breaks the tie
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert np.array_equal(fp8.encode(up), np.arange(1, 127, dtype=np.uint8))
    assert np.array_equal(fp8.encode(dn), np.arange(0, 126, dtype=np.uint8))


def test_encode_saturation_signs_nan():
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf],
                   dtype=np.float32)
    assert np.all(fp8.encode(big) == 0x7E)
    assert np.all(fp8.encode(-big) == 0xFE)
    assert fp8.encode(np.float32(-0.0)) == 0x80
    assert fp8.encode(np.float32(0.0)) == 0x00
    assert fp8.encode(np.float32(-1e-9)) == 0x80
    assert fp8.encode(np.float32(np.nan)) == 0x7F


@pytest.mark.parametrize("val,code", [(2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01),
                                      (2.0 ** -9, 0x01), (1.0625, 0x38),
                                      (1.1875, 0x3A), (240.0, 0x77)])
def test_encode_handpicked(val, code):
    # 2^-10 is halfway between 0 and 2^-9: tie to the even code 0x00;
    # 3*2^-11 is above that midpoint: 0x01; 1.0625 is halfway between
    # 1.0 (0x38) and 1.125 (0x39): even 0x38; 1.1875 halfway between
    # 1.125 (0x39) and 1.25 (0x3A): even 0x3A; 240 = 1.875 * 2^7 = 0x77.
    assert fp8.encode(np.float32(val)) == code
