"""e4m3 and bfloat16 number formats, written out from their definitions.

OCP E4M3FN (the "e4m3" of "ZYFA: Fast and Accurate FP8 Attention on AMD
MI355X", section "Precision and Underflow of FP8 Probabilities", footnote 7;
range from the FP8 GEMM on CDNA4 blog, section 2.1):

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
* exponent field 1..15: value = (1 + m/8) * 2^(e - 7); field 0: subnormal,
  value = m/8 * 2^-6 = m * 2^-9.
* no infinities; code 0x7F / 0xFF is NaN, so the largest finite value is
  0x7E = 1.75 * 2^8 = 448.
* read as an integer, a positive code grows by 8 for each doubling of the
  value: 1 -> 56, 2 -> 64, 4 -> 72, and 60 -> 1.5 (footnote 7).
* smallest normal 2^-6; values below 2^-10 (half the smallest subnormal)
  round to zero.

Rounding is round-to-nearest, ties to even (blog section 2.3), and encoding
saturates at +-448 (values beyond the largest finite value clamp to it rather
than becoming NaN), so ``e4m3_encode`` is total on finite inputs.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode e4m3 codes (any integer array, values 0..255) to float64."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    subnormal = man * 2.0 ** -9
    normal = (8 + man) * np.ldexp(1.0, exp - 10)  # (1 + m/8) * 2^(e-7)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# The 127 finite non-negative e4m3 values, ascending; index == code (0x00..0x7E).
_POSITIVE = e4m3_decode(np.arange(127))
assert np.all(np.diff(_POSITIVE) > 0)


def e4m3_encode(x):
    """Round float values to e4m3 codes (uint8): nearest value, ties to the even
    code, saturating at +-448. NaN maps to 0x7F. The sign bit is kept for values
    that round to zero (-0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POSITIVE, mag, side="left")  # first value >= mag
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = mag - _POSITIVE[lo]
    d_hi = _POSITIVE[hi] - mag
    # Among the two neighbours, take the nearer; on a tie take the even code.
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(mag == _POSITIVE[hi], hi, code)
    code = code | (np.signbit(x).astype(np.int64) << 7)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (ties to even); returns the uint16 bit patterns.

    A bfloat16 is the upper half of a float32. Of the two bfloat16 values that
    bracket x (its truncation t and t + 1 ulp), take the nearer; on a tie take
    the one whose last bit is 0. NaN stays a quiet NaN."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    trunc = bits >> 16
    rest = bits & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((trunc & 1) == 1))
    out = trunc + up.astype(np.uint64)
    out = np.where(np.isnan(x), (trunc | 0x40), out)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 value, returned as float64."""
    return bf16_bits_to_f64(f32_to_bf16_bits(x))
