"""Scale file (calibrate once, reuse): parsing, aliases, validation and the saved numbers.

The printed example of vLLM docs "FP8 ViT Encoder Attention", section "Scale file
format" (tests/golden/scale_file_example.json) must parse, with the q_scale/k_scale/v_scale
aliases accepted; the numbers written for a calibrated layer must be the oracle's static
amax, fp32(window max * margin) (oracle.static_amax), and survive a write/read unchanged.
No GPU: explicit window-amax triples and a zeroed host copy of a layer state stand in
for calibrated layers.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_dynamic_scaled_amd import scale_file as sf
from fp8_dynamic_scaled_amd.api import STATE_DTYPE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_file_example.json")


def _example():
    with open(GOLDEN) as f:
        return json.load(f)["layers"]


def test_pages_example_parses_to_static_amax():
    got = sf.parse_scale_file(_example())
    assert got == {"visual.blocks.0.attn.attn": (224.0, 198.0, 210.0),
                   "visual.blocks.1.attn.attn": (218.0, 195.0, 207.0)}
    # the reading: each number is A, scale = A / 448 -- the example's 224 is scale 0.5
    assert oracle.scale_pair(224.0) == (0.5, 2.0)


def test_aliases_are_accepted_and_must_agree():
    ex = _example()
    aliased = {name: {f"{t}_scale": v for t, v in vals.items()} for name, vals in ex.items()}
    assert sf.parse_scale_file(aliased) == sf.parse_scale_file(ex)
    both = {"l": {"q": 1.0, "q_scale": 1.0, "k": 2.0, "v_scale": 3.0}}
    assert sf.parse_scale_file(both) == {"l": (1.0, 2.0, 3.0)}
    with pytest.raises(sf.ScaleFileError, match="disagree"):
        sf.parse_scale_file({"l": {"q": 1.0, "q_scale": 2.0, "k": 2.0, "v": 3.0}})


@pytest.mark.parametrize("bad,needle", [
    ([1, 2], "JSON object"),
    ({"l": [1.0, 2.0, 3.0]}, "expected an object"),
    ({"l": {"q": 1.0, "k": 2.0}}, "missing 'v'"),
    ({"l": {"q": 1.0, "k": 2.0, "v": 3.0, "w": 4.0}}, "unknown keys"),
    ({"l": {"q": -1.0, "k": 2.0, "v": 3.0}}, ">= 0"),
    ({"l": {"q": float("nan"), "k": 2.0, "v": 3.0}}, "finite"),
    ({"l": {"q": float("inf"), "k": 2.0, "v": 3.0}}, "finite"),
    ({"l": {"q": "1", "k": 2.0, "v": 3.0}}, "not a number"),
    ({"l": {"q": True, "k": 2.0, "v": 3.0}}, "not a number"),
])
def test_invalid_files_are_rejected(bad, needle):
    with pytest.raises(sf.ScaleFileError, match=needle):
        sf.parse_scale_file(bad)


def test_saved_numbers_are_the_oracle_static_amax():
    rng = np.random.default_rng(11)
    # window maxima are bf16 magnitudes (exact amax of bf16 tensors): draw bf16 patterns
    bits = rng.integers(0, 0x7F80, size=(64, 3), dtype=np.uint16)
    wins = oracle.bf16_bits_to_f64(bits)
    amax = {f"layer{i}": tuple(float(x) for x in row) for i, row in enumerate(wins)}
    for margin in (1.5, 1.0, 1.3, 2.0):
        got = sf.entries(amax, margin)
        for name, trip in amax.items():
            want = oracle.static_amax(list(trip), float(np.float32(margin)))
            assert [got[name][t] for t in sf.TENSORS] == [float(x) for x in want], (name, margin)


def test_write_read_round_trip_is_exact(tmp_path):
    rng = np.random.default_rng(5)
    amax = {f"visual.blocks.{i}.attn.attn": tuple(float(np.float32(x)) for x in rng.gamma(2.0, 40.0, 3))
            for i in range(27)}
    path = str(tmp_path / "scales.json")
    written = sf.save_scale_file(path, amax, margin=1.5)
    back = sf.load_scale_file(path)
    assert set(back) == set(amax)
    for name in amax:
        assert back[name] == tuple(written[name][t] for t in sf.TENSORS)
        want = oracle.static_amax(list(amax[name]), 1.5)
        assert back[name] == tuple(float(x) for x in want)
    with open(path) as f:
        raw = json.load(f)
    assert set(raw["visual.blocks.0.attn.attn"]) == {"q", "k", "v"}


def test_margin_and_amax_are_validated():
    with pytest.raises(sf.ScaleFileError, match="margin"):
        sf.entries({"l": (1.0, 1.0, 1.0)}, 0.0)
    with pytest.raises(sf.ScaleFileError, match="margin"):
        sf.entries({"l": (1.0, 1.0, 1.0)}, float("nan"))
    with pytest.raises(sf.ScaleFileError, match=">= 0"):
        sf.entries({"l": (1.0, -2.0, 1.0)})
    with pytest.raises(sf.ScaleFileError, match=r"\(q, k, v\)"):
        sf.entries({"l": (1.0, 2.0)})


def test_an_uncalibrated_state_cannot_be_saved(tmp_path):
    st = torch.zeros(STATE_DTYPE.itemsize, dtype=torch.uint8)     # host copy of a fresh state
    with pytest.raises(sf.ScaleFileError, match="no dynamic forward"):
        sf.window_amax(st)
    rec = np.zeros(1, dtype=STATE_DTYPE)
    rec["count"] = 16
    rec["amax"] = [3.5, 2.25, 448.0]
    st = torch.from_numpy(rec.view(np.uint8).copy())
    assert sf.window_amax(st) == (3.5, 2.25, 448.0)
    data = sf.save_scale_file(str(tmp_path / "s.json"), {"l": st})
    assert data == {"l": {"q": 5.25, "k": 3.375, "v": 672.0}}
    assert all(math.isfinite(x) for x in data["l"].values())
