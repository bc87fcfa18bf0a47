"""Per-tensor amax, the 16-slot amax ring and the scale rule (oracle; test only).

Sources:
  * vLLM docs "FP8 ViT Encoder Attention", section "Usage": without a scale file the
    scale of every forward is driven by a circular buffer of the 16 most recent observed
    Q/K/V amax values; with static scales a calibrated value is reused; saved scales are
    multiplied by a margin whose default is 1.5.
  * Same page, section "Scale file format": one q, k, v triple per attention layer.
  * The varlen backend of the Korean wiki rewrite ("Requirements") uses one scale per
    tensor ("pertensor").

Readings where the pages are silent:
  * amax is per tensor over the whole packed batch (all sequences, heads, channels).
  * Ring slot of dynamic forward f is f mod 16; empty slots hold 0; the current forward's
    amax is inserted before its own scale is computed; A = max over the 16 slots.
  * scale = A / 448 and inv = 448 / A, each rounded once to binary32 (448 = E4M3 max);
    A is floored at 2^-64 so that inv stays finite and 0 * inv is never NaN.
  * Static: A = binary32(calibrated amax * margin).
  * One ring per tensor per layer; forwards that skip FP8 do not observe.
"""

import numpy as np

from .numerics import bf16_bits_to_f64, round_f32

RING_SLOTS = 16
E4M3_MAX = 448.0
SCALE_FLOOR = 2.0 ** -64


def amax_bf16(bits):
    """max |x| over a bf16 tensor given as uint16 bit patterns; 0.0 for an empty one."""
    x = bf16_bits_to_f64(bits)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x)))


def amax_bf16_bits(bits):
    """Same value as amax_bf16, computed on the bit patterns: for finite bf16 values the
    pattern with the sign bit cleared orders exactly like |x|, so max|x| is the value of
    the largest such pattern. Used for large tensors (no float64 copy)."""
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    if b.size == 0:
        return 0.0
    m = np.uint32(np.max(b & np.uint16(0x7FFF)))
    return float(np.array([m << np.uint32(16)], dtype=np.uint32).view(np.float32)[0])


def scale_pair(amax):
    """(scale, inv) for one tensor from its window/static amax A (a binary32 value).

    float64 division of two binary32 values followed by rounding to binary32 is the
    correctly rounded binary32 quotient (53 >= 2*24 + 2), so this is exactly the
    IEEE single-precision division.
    """
    a = max(float(amax), SCALE_FLOOR)
    scale = float(round_f32(a / E4M3_MAX))
    inv = float(round_f32(E4M3_MAX / a))
    return scale, inv


def static_amax(calibrated, margin=1.5):
    """A = binary32(calibrated amax * margin) for q, k, v (margin default 1.5)."""
    cal = round_f32(np.asarray(calibrated, dtype=np.float64))
    m = float(round_f32(margin))
    return [float(v) for v in round_f32(cal * m)]


class AmaxRing:
    """Circular buffer of the last 16 observed amax values of Q, K and V (one layer)."""

    def __init__(self):
        self.slots = np.zeros((3, RING_SLOTS), dtype=np.float64)
        self.count = 0

    def update(self, amax_qkv):
        """Insert this forward's (q, k, v) amax and return the window maxima A."""
        slot = self.count % RING_SLOTS
        for t in range(3):
            self.slots[t, slot] = float(amax_qkv[t])
        self.count += 1
        return [float(np.max(self.slots[t])) for t in range(3)]
