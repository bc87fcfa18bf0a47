"""Pins of the oracle's E4M3 codec against things other than itself.

* the published E4M3 table values (tests/golden/e4m3_spec_values.txt, OCP OFP8 spec),
* brute-force nearest over the 127 non-negative finite values (exhaustive over every
  bf16 pattern under several multipliers),
* torch's float8_e4m3fn conversion (a library codec: single rounding, RNE, NaN above
  the saturation point, so it is compared after clamping to +-448),
* round trip, monotonicity and the relative error bound of a 3-bit mantissa.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode, round_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_bf16_finite_f64():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_bits_to_f64(bits)
    return x[np.isfinite(x)]


def test_published_table_values():
    table = oracle.e4m3_decode_table()
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code_s, val_s = line.split()
            code = int(code_s, 16)
            val = float(val_s)
            if math.isnan(val):
                assert math.isnan(table[code])
            else:
                assert table[code] == val
                assert math.copysign(1, table[code]) == math.copysign(1, val)
                # and the encoder maps the value back to that code
                assert int(e4m3_encode(np.array([val]))[0]) == code


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    vals = e4m3_decode(codes)
    back = e4m3_encode(vals)
    assert np.array_equal(back, codes)


def test_monotone_and_max():
    codes, vals = oracle.e4m3_finite_values()
    assert codes.size == 127
    assert np.all(np.diff(vals) > 0)
    assert vals[-1] == 448.0 and vals[0] == 0.0
    y = np.linspace(-500, 500, 200001)
    enc = e4m3_decode(e4m3_encode(y))
    assert np.all(np.diff(enc) >= 0)


def _brute_force_nearest(y):
    """Nearest non-negative E4M3 value by exhaustive search; ties -> even code."""
    codes, vals = oracle.e4m3_finite_values()
    a = np.abs(y)
    out = np.empty(y.shape, dtype=np.uint8)
    for s in range(0, a.size, 65536):
        blk = a[s:s + 65536]
        dist = np.abs(blk[:, None] - vals[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        # among equal-distance candidates prefer an even code (mantissa LSB 0)
        even = cand & ((codes[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        c = codes[pick]
        c = np.where(blk >= 448.0, 0x7E, c)
        out[s:s + 65536] = c
    return out | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


@pytest.mark.parametrize("inv", [1.0, 2.0 ** -3, 448.0 / 20.0, 448.0 / 3.0, 0.7071067690849304,
                                 448.0 / 7.5, 2.0 ** 7 + 0.25, 1.0 / 3.0])
def test_exhaustive_bf16_vs_brute_force(inv):
    inv = float(round_f32(inv))
    x = _all_bf16_finite_f64()
    y = round_f32(x * inv)
    got = e4m3_encode(y)
    want = _brute_force_nearest(y)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_exhaustive_bf16_vs_torch_float8(seed):
    rng = np.random.default_rng(seed)
    invs = round_f32(np.exp(rng.uniform(-8, 8, size=16)))
    x = _all_bf16_finite_f64()
    for inv in invs:
        y = round_f32(x * float(inv))
        got = e4m3_encode(y)
        t = torch.from_numpy(np.clip(y, -448.0, 448.0).astype(np.float32))
        want = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, want), f"inv={inv}"


def test_special_values():
    cases = [(448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (math.inf, 0x7E),
             (-math.inf, 0xFE), (-448.0, 0xFE), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80),
             (1.5 * 2.0 ** -9, 0x02), (17.0, 0x58), (19.0, 0x5A), (1.0625, 0x38),
             (1.0625 + 2.0 ** -20, 0x39), (0.0, 0x00), (-0.0, 0x80), (-1e-6, 0x80),
             (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (240.0, 0x77), (256.0, 0x78)]
    for y, code in cases:
        assert int(e4m3_encode(np.array([y]))[0]) == code, (y, hex(code))
    assert int(e4m3_encode(np.array([math.nan]))[0]) & 0x7F == 0x7F


def test_error_bound():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(2.0 ** -6, 448, 100000), rng.uniform(0, 2.0 ** -6, 100000)])
    y = np.concatenate([y, -y])
    err = np.abs(e4m3_decode(e4m3_encode(y)) - y)
    big = np.abs(y) >= 2.0 ** -6
    assert np.all(err[big] <= 2.0 ** -4 * np.abs(y[big]))
    assert np.all(err[~big] <= 2.0 ** -10)
