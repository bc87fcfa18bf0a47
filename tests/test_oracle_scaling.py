"""Pins of the oracle's amax, ring and scale rule.

* scale/inv against exact rational arithmetic (fractions) rounded to binary32 by an
  independent routine, exhaustively over every non-negative finite bf16 value of A,
* the pages' worked scale-file numbers and default margin
  (tests/golden/scale_file_example.json),
* closed-form ring trajectories (window maximum of the last 16 observations),
* amax against an integer maximum over the bf16 bit patterns with the sign cleared.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _round_fraction_to_f32(q: Fraction) -> float:
    """Correctly rounded (ties to even) binary32 value of a positive rational."""
    assert q > 0
    # exponent e with 2^e <= q < 2^(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    if Fraction(2) ** (e + 1) <= q:
        e += 1
    e_eff = max(e, -126)                     # subnormal quantum below 2^-126
    quantum = Fraction(2) ** (e_eff - 23)
    n = q / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * quantum
    if val >= Fraction(2) ** 128:
        return float("inf")
    return float(val)


def test_scale_pair_exhaustive_vs_fractions():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)        # +0 .. largest finite bf16
    amax = oracle.bf16_bits_to_f64(bits)
    assert amax.size == 32640
    for a in amax:
        s, inv = oracle.scale_pair(a)
        a_eff = Fraction(max(float(a), 2.0 ** -64))
        assert s == _round_fraction_to_f32(a_eff / 448)
        assert inv == _round_fraction_to_f32(448 / a_eff)
        assert np.isfinite(inv) and inv > 0


def test_scale_file_worked_example():
    with open(os.path.join(GOLDEN, "scale_file_example.json")) as f:
        g = json.load(f)
    layer0 = g["layers"]["visual.blocks.0.attn.attn"]
    s, inv = oracle.scale_pair(layer0["q"])
    assert s == 0.5 and inv == 2.0                      # 224 = 448 / 2
    for key in ("k", "v"):
        a = layer0[key]
        s, inv = oracle.scale_pair(a)
        assert s == _round_fraction_to_f32(Fraction(a) / 448)
        assert inv == _round_fraction_to_f32(Fraction(448) / Fraction(a))
    # static mode: A = fp32(calibrated amax * margin); margin default 1.5
    assert g["margin_default"] == 1.5
    assert oracle.static_amax([2.0, 4.0, 1.0], g["margin_default"]) == [3.0, 6.0, 1.5]
    # a calibrated amax of 224/1.5 reproduces the file's q entry: binary32(224/1.5) times 1.5
    # is exactly 224 - 2^-17, half a binary32 step below 224, a tie that binary32 rounding
    # settles on 224 (even significand); without that rounding A would stay 224 - 2^-17
    c = float(np.float32(224.0 / 1.5))
    assert c * 1.5 == 224.0 - 2.0 ** -17
    A = oracle.static_amax([224.0 / 1.5, 1.0, 1.0])[0]
    assert A == 224.0


def test_zero_amax_floor():
    s, inv = oracle.scale_pair(0.0)
    assert inv == float(np.float32(448.0 * 2.0 ** 64))
    assert np.isfinite(inv) and 0.0 * inv == 0.0


def test_ring_window_closed_form():
    ring = oracle.AmaxRing()
    obs = [float(20 - f) for f in range(20)]            # 20, 19, ..., 1
    got = [ring.update([o, o / 2, o / 4])[0] for o in obs]
    for f in range(20):
        want = max(obs[max(0, f - 15):f + 1])           # last 16 observations
        assert got[f] == want
    assert got[:16] == [20.0] * 16 and got[16] == 19.0 and got[19] == 16.0


def test_ring_random_trajectory_matches_window_max():
    rng = np.random.default_rng(7)
    ring = oracle.AmaxRing()
    hist = []
    for f in range(50):
        a = rng.uniform(0, 10, size=3)
        hist.append(a)
        A = ring.update(a)
        window = np.array(hist[max(0, f - 15):])
        assert np.array_equal(np.array(A), window.max(axis=0))
    assert ring.count == 50


@pytest.mark.parametrize("seed", range(3))
def test_amax_vs_integer_bits(seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 65536, size=100000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]               # finite only
    a = oracle.amax_bf16(bits)
    m = int(np.max(bits & 0x7FFF))
    assert a == float(oracle.bf16_bits_to_f64(np.array([m], dtype=np.uint16))[0])
    assert oracle.amax_bf16(np.zeros(0, np.uint16)) == 0.0
    # the bit-pattern formulation gives the same value, including -0.0 and subnormals
    assert oracle.amax_bf16_bits(bits) == a
    special = np.array([0x8000, 0x0001, 0x8002, 0x0000], dtype=np.uint16)
    assert oracle.amax_bf16_bits(special) == oracle.amax_bf16(special) == 2.0 ** -132
    assert oracle.amax_bf16_bits(np.zeros(0, np.uint16)) == 0.0


def test_quantize_saturates_under_static_small_margin():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000) * 4
    bits = np.frombuffer(x.astype(np.float32).tobytes(), dtype=np.uint32) >> 16
    bits = bits.astype(np.uint16)
    amax = oracle.amax_bf16(bits)
    A = oracle.static_amax([amax], 0.5)[0]
    _, inv = oracle.scale_pair(A)
    codes = oracle.quantize_bf16(bits, inv)
    xv = oracle.bf16_bits_to_f64(bits)
    over = np.abs(oracle.round_f32(xv * inv)) >= 448
    assert over.any()
    assert np.all((codes[over] & 0x7F) == 0x7E)
    # dynamic scale never saturates beyond the max: no code above 448 in magnitude
    _, inv_d = oracle.scale_pair(amax)
    cd = oracle.quantize_bf16(bits, inv_d)
    assert np.all((cd & 0x7F) <= 0x7E)
    assert (cd & 0x7F).max() == 0x7E                  # the amax element maps to 448


@pytest.mark.parametrize("seed", range(3))
def test_quantize_vs_torch_library(seed):
    """quantize_bf16 == torch: bf16 -> fp32 multiply by inv -> clamp -> float8_e4m3fn."""
    import torch
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(200000, generator=g) * 10 ** (seed - 1)).to(torch.bfloat16)
    x[:5] = torch.tensor([0.0, -0.0, 1e-30, -3e38, 3e38], dtype=torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    for amax in (oracle.amax_bf16(bits), 1e-3, 7.25, 1e30):
        _, inv = oracle.scale_pair(float(np.float32(amax)))
        y = x.float() * torch.tensor(inv, dtype=torch.float32)
        want = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.quantize_bf16(bits, inv), want)

