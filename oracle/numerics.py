"""Exact conversions between bit patterns and float64 (oracle; test infrastructure only).

bf16 is the top half of an IEEE binary32, so a bf16 bit pattern b denotes exactly the
binary32 value whose bits are b << 16; every such value is exactly a float64.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """float64 values of bf16 bit patterns (uint16 array), exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 (round to nearest, ties to even), return uint16 bits.

    Rounds in two exact steps: the float64 value is first rounded to binary32 only if
    it is already a binary32 value; otherwise the bf16 rounding is done directly on the
    float64 by scaling to the bf16 quantum of its binade. Used only by input generators
    and tests to build bf16 fixtures.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    o = out.reshape(-1)
    for i, v in enumerate(flat):
        o[i] = _f64_to_bf16_scalar(float(v))
    return out


def _f64_to_bf16_scalar(v):
    import math
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a == 0.0:
        return sign
    # bf16: 8 significant bits, exponent range of binary32, subnormal quantum 2^-133.
    m, e = math.frexp(a)          # a = m * 2^e, m in [0.5, 1)
    q_exp = max(e - 8, -133)      # quantum of the binade (8 significant bits)
    n = a / math.ldexp(1.0, q_exp)
    r = round(n)                  # Python round: ties to even
    val = math.ldexp(float(r), q_exp)
    if val >= math.ldexp(1.0, 128):
        return sign | 0x7F80      # overflow to infinity
    bits32 = np.array([val], dtype=np.float32).view(np.uint32)[0]
    return sign | int(bits32 >> 16)


def round_f32(x):
    """Round float64 values to the nearest binary32 (ties to even), returned as float64.

    numpy's float64 -> float32 cast is the IEEE round-to-nearest-even conversion;
    magnitudes beyond the binary32 range become +-inf.
    """
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
