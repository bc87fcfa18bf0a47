"""OCP E4M3 ("E4M3FN") codec written from the format definition (oracle; test only).

The Ascend chapter "5.4 昇腾量化与 KV Cache 优化" (section 4, FP8 quantisation) names the
two FP8 formats, E4M3 and E5M2; the attention path uses E4M3. The pages do not spell the
format out, so it is taken from the OCP 8-bit floating point specification:
  * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  * exponent field 0 encodes subnormals m * 2^-9 (m = 1..7) and zero;
  * exponent field e = 1..15 encodes (1 + m/8) * 2^(e-7), except that e = 15, m = 7
    (0x7F / 0xFF) is NaN; there are no infinities, so the largest magnitude is
    (1 + 6/8) * 2^8 = 448 (0x7E).
Encoding (the reading used throughout, since the pages fix no rounding rule): round to
nearest with ties to even on the value grid, saturate magnitudes >= 448 (and +-inf) to
+-448, keep the sign of zero and of values that round to zero, NaN -> 0x7F | sign.
"""

import math

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6      # smallest normal binade is [2^-6, 2^-5)
_MANT_BITS = 3


def _decode_scalar(code):
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_DECODE = np.array([_decode_scalar(c) for c in range(256)], dtype=np.float64)


def e4m3_decode_table():
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    return _DECODE.copy()


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array) as float64."""
    return _DECODE[np.asarray(codes, dtype=np.uint8)]


def e4m3_finite_values():
    """The 127 non-negative finite E4M3 values with their codes, ascending by value."""
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)
    return codes, _DECODE[codes]


def e4m3_encode(y):
    """Encode real values (float64 array) to E4M3 codes, RNE, saturating.

    For finite |y| < 448: the binade exponent is e = max(floor(log2|y|), -6) and the
    spacing of representable values there is 2^(e-3); |y| is divided by that spacing
    (exact: a power of two), rounded to an integer with ties to even, and multiplied
    back. A result of 2^(e+1) (integer 16) simply belongs to the next binade.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))
    a = np.abs(y)
    out = np.zeros(y.shape, dtype=np.uint8)

    is_nan = np.isnan(y)
    is_sat = (~is_nan) & (a >= E4M3_MAX)          # includes +-inf
    is_fin = (~is_nan) & (~is_sat)

    af = a[is_fin]
    # floor(log2 af) exactly: frexp gives af = f * 2^ex with f in [0.5, 1).
    _, ex = np.frexp(af)
    e = np.maximum(ex.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    spacing_exp = e - _MANT_BITS
    n = np.rint(np.ldexp(af, -spacing_exp))        # ties to even
    val = np.ldexp(n, spacing_exp)                 # the representable value, < 448 + spacing

    # Turn the representable value into its code.
    codes = np.zeros(af.shape, dtype=np.int64)
    nz = val > 0
    v = val[nz]
    _, vex = np.frexp(v)
    ve = vex.astype(np.int64) - 1                  # exact binade of the value
    sub = ve < _MIN_NORMAL_EXP
    c = np.empty(v.shape, dtype=np.int64)
    # subnormal: v = m * 2^-9
    c[sub] = np.ldexp(v[sub], 9).astype(np.int64)
    # normal: v = (1 + m/8) * 2^ve, exponent field ve + 7
    vn = v[~sub]
    ven = ve[~sub]
    mant = (np.ldexp(vn, -ven) - 1.0) * 8.0
    c[~sub] = ((ven + 7) << 3) | mant.astype(np.int64)
    codes[nz] = c
    out[is_fin] = codes.astype(np.uint8)
    out[is_sat] = 0x7E
    out[is_nan] = 0x7F
    return out | sign
