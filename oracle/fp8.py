"""OCP FP8 e4m3fn codec, written from the format's bit definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Format (OCP 8-bit floating point, E4M3 "fn" variant; the indexer-K cache and
the quantised query use it -- GLM-5.3 KV/indexer cache budget article, section
on the two caches' byte accounts: 128 FP8 key bytes plus one FP32 scale per
128-element block):

* bit 7 is the sign, bits 6..3 the biased exponent E (bias 7), bits 2..0 the
  mantissa M;
* E == 0: subnormal, value = M/8 * 2**-6;
* E == 15 and M == 7: NaN (there is no infinity);
* otherwise value = (1 + M/8) * 2**(E - 7); the largest finite magnitude is
  1.75 * 2**8 = 448 (code 0x7E).

Encoding rounds to the nearest representable value, ties to the code with an
even mantissa (round-to-nearest-even), and saturates magnitudes above 448 to
448 ("satfinite").

Pins (tests/test_oracle_fp8.py): every one of the 256 codes against the closed
form above and against torch's float8_e4m3fn -> float32 conversion; spot
values 0x7E = 448, 0x08 = 2**-6, 0x01 = 2**-9; the encoder against torch's
float32 -> float8_e4m3fn cast on in-range inputs, including every exact
midpoint between adjacent codes.
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode(codes):
    """Decode e4m3fn bytes to float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1 == 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def positive_code_values():
    """Values of the finite non-negative codes 0x00..0x7E, in code order.

    The format is monotonic in the code for non-negative values, so this
    array is sorted ascending.
    """
    return decode(np.arange(0, 0x7F, dtype=np.uint8))


def encode(x):
    """Round float values to e4m3fn codes: nearest value, ties to even
    mantissa, magnitudes above 448 saturate to 448, NaN -> 0x7F.

    The sign of the input (including -0.0) becomes the sign bit, so a negative
    value that rounds to zero encodes as 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    vals = positive_code_values()                   # 127 ascending values
    mag = np.abs(x)
    nan = np.isnan(x)
    mag_c = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))
    hi = np.searchsorted(vals, mag_c, side="left")  # first value >= mag
    hi = np.clip(hi, 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_hi = vals[hi] - mag_c
    d_lo = mag_c - vals[lo]
    pick_lo = d_lo < d_hi
    tie = d_lo == d_hi
    # On a tie the two neighbours differ by one code; take the even one.
    pick_lo = np.where(tie, (lo % 2) == 0, pick_lo)
    code = np.where(pick_lo, lo, hi).astype(np.int64)
    code = np.where(mag_c == vals[hi], hi, code)    # exact hit
    negative = np.signbit(x)
    code = np.where(negative, code | 0x80, code)
    code = np.where(nan, NAN_CODE, code)
    return code.astype(np.uint8)
