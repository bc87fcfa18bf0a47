"""Calibrate once, reuse: the static scale file.

vLLM docs "FP8 ViT Encoder Attention", section "Usage" (repeated in the Korean wiki
rewrite, "Calibrate-Once, Reuse"): a calibration run uses dynamic scaling for 16 forwards
over representative data, then writes the learned per-layer values, multiplied by a
safety margin (default 1.5), to a JSON file; serving loads the file and runs every layer
with static scales, with no amax observation per forward. Section "Scale file format":
one JSON object per attention layer, keyed by the layer's name, holding one number for
each of "q", "k" and "v"; "q_scale", "k_scale" and "v_scale" are accepted as aliases.

Reading of the numbers (the pages print an example but do not define it further): each
is the per-tensor A of static mode -- the layer's dynamic window maximum (max of the last
16 observed amax values) times the margin -- and the FP8 scale derived from it is A/448,
so the printed 224.0 means scale 0.5. Saving multiplies in fp32, exactly as the library's
static-scale kernel does with a margin; loading hands the numbers back unchanged (static
mode with margin 1), so a saved-then-loaded layer quantises exactly as a layer built with
static_amax = window maximum and margin = 1.5.

Host I/O only: the numbers come from a layer's device state (one copy of the state
bytes) and go to AttentionLayer(static_amax=..., margin=1.0); nothing here runs per
forward.
"""
import json
import math
from typing import Dict, Mapping, Sequence, Tuple, Union

import numpy as np

from .api import DEFAULT_MARGIN, AttentionLayer, read_state

CALIBRATION_FORWARDS = 16          # dynamic forwards per layer before the file is written
TENSORS = ("q", "k", "v")
_ALIASES = {"q": "q_scale", "k": "k_scale", "v": "v_scale"}

Triple = Tuple[float, float, float]


class ScaleFileError(ValueError):
    """A scale file (or a calibrated layer) that cannot be used."""


def _fp32(x: float) -> float:
    return float(np.float32(x))


def window_amax(layer_or_state) -> Triple:
    """The (q, k, v) window maxima of a layer that has run dynamic forwards: the A that
    its last dynamic forward used (max over the 16-slot ring, this forward included)."""
    state = layer_or_state.state if isinstance(layer_or_state, AttentionLayer) else layer_or_state
    s = read_state(state)
    if int(s["count"]) == 0:
        raise ScaleFileError("the layer has run no dynamic forward; nothing to calibrate from")
    return tuple(float(a) for a in s["amax"])


def entries(amax: Mapping[str, Sequence[float]], margin: float = DEFAULT_MARGIN
            ) -> Dict[str, Dict[str, float]]:
    """{layer: {"q": A, "k": A, "v": A}} with A = fp32(window max * margin)."""
    m = np.float32(margin)
    if not (math.isfinite(float(m)) and float(m) > 0):
        raise ScaleFileError(f"margin must be finite and > 0, got {margin!r}")
    out = {}
    for name, trip in amax.items():
        if len(trip) != 3:
            raise ScaleFileError(f"{name}: need (q, k, v) amax, got {trip!r}")
        vals = {}
        for t, a in zip(TENSORS, trip):
            a32 = np.float32(a)
            if not (math.isfinite(float(a32)) and float(a32) >= 0):
                raise ScaleFileError(f"{name}.{t}: amax must be finite and >= 0, got {a!r}")
            vals[t] = float(np.float32(a32 * m))
        out[str(name)] = vals
    return out


def save_scale_file(path: str, layers: Mapping[str, Union[AttentionLayer, Sequence[float]]],
                    margin: float = DEFAULT_MARGIN) -> Dict[str, Dict[str, float]]:
    """Write the scale file for calibrated layers ({name: AttentionLayer or state, or an
    explicit (q, k, v) window-amax triple}). Returns what was written."""
    amax = {}
    for name, x in layers.items():
        if isinstance(x, (tuple, list)):
            amax[name] = tuple(float(v) for v in x)
        else:
            amax[name] = window_amax(x)
    data = entries(amax, margin)
    with open(path, "w") as f:
        json.dump(data, f, indent=2)
        f.write("\n")
    return data


def parse_scale_file(obj) -> Dict[str, Triple]:
    """{layer: (A_q, A_k, A_v)} from the parsed JSON of a scale file (aliases resolved)."""
    if not isinstance(obj, dict):
        raise ScaleFileError("a scale file is a JSON object keyed by layer name")
    out = {}
    for name, val in obj.items():
        if not isinstance(val, dict):
            raise ScaleFileError(f"{name}: expected an object with q/k/v numbers")
        unknown = set(val) - set(TENSORS) - set(_ALIASES.values())
        if unknown:
            raise ScaleFileError(f"{name}: unknown keys {sorted(unknown)}")
        trip = []
        for t in TENSORS:
            have = [k for k in (t, _ALIASES[t]) if k in val]
            if not have:
                raise ScaleFileError(f"{name}: missing {t!r} (or {_ALIASES[t]!r})")
            nums = [val[k] for k in have]
            for x in nums:
                if isinstance(x, bool) or not isinstance(x, (int, float)):
                    raise ScaleFileError(f"{name}.{t}: not a number: {x!r}")
            if len(nums) == 2 and _fp32(nums[0]) != _fp32(nums[1]):
                raise ScaleFileError(f"{name}: {t!r} and {_ALIASES[t]!r} disagree")
            a = _fp32(nums[0])
            if not (math.isfinite(a) and a >= 0):
                raise ScaleFileError(f"{name}.{t}: must be finite and >= 0, got {nums[0]!r}")
            trip.append(a)
        out[str(name)] = tuple(trip)
    return out


def load_scale_file(path: str) -> Dict[str, Triple]:
    """Read a scale file: {layer: (A_q, A_k, A_v)}, each A the static-mode amax."""
    with open(path) as f:
        return parse_scale_file(json.load(f))


def static_layers(path_or_scales, device=None) -> Dict[str, AttentionLayer]:
    """One static-scale AttentionLayer per entry of a scale file (margin 1: the file's
    numbers already carry the calibration margin)."""
    scales = (load_scale_file(path_or_scales) if isinstance(path_or_scales, str)
              else dict(path_or_scales))
    return {name: AttentionLayer(device, static_amax=trip, margin=1.0)
            for name, trip in scales.items()}
