"""Calibrate once on the GPU, save the scale file, load it, reuse it (vLLM docs "FP8 ViT
Encoder Attention", sections "Usage" and "Scale file format").

Two layers run 19 dynamic forwards each; the first draw is the largest and has left the
16-slot window by the end, so the file must hold the window maximum, not the all-time
one. The numbers written must be the oracle's fp32(window max * 1.5); a layer loaded from
the file must produce the same bytes as a static layer built from the window maximum
with margin 1.5, carry the oracle's scales, and match the oracle's FP8 attention.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_dynamic_scaled_amd as fa
from fp8_dynamic_scaled_amd import scale_file as sf
from workloads import random_varlen

from parity_util import amax_exact, bf16_to_f64, compare, oracle_fp8_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
SM = fa.default_softmax_scale()


def say(msg):
    print(msg, flush=True)


def _cu_dev(cu):
    return torch.tensor(cu, dtype=torch.int32, device=DEV)


def test_calibrate_save_load_reuse(tmp_path):
    H, lens = 2, [300, 77]
    names = ["visual.blocks.0.attn.attn", "visual.blocks.1.attn.attn"]
    layers = {n: fa.AttentionLayer(DEV) for n in names}
    rings = {n: oracle.AmaxRing() for n in names}
    window, alltime = {}, {n: [0.0, 0.0, 0.0] for n in names}
    forwards = sf.CALIBRATION_FORWARDS + 3
    for f in range(forwards):
        for i, name in enumerate(names):
            scale = 3.0 if f == 0 else 1.0 + 0.05 * (f % 4)
            q, k, v, cu = random_varlen(lens, H, seed=500 + 50 * i + f, device=DEV,
                                        outliers=True, scale=scale)
            layers[name](q, k, v, _cu_dev(cu), cu)
            a = [amax_exact(t) for t in (q, k, v)]
            alltime[name] = [max(x, y) for x, y in zip(alltime[name], a)]
            window[name] = rings[name].update(a)
    torch.cuda.synchronize()
    say(f"calibrated {len(names)} layers over {forwards} forwards; window max {window}")
    for name in names:
        assert int(fa.read_state(layers[name].state)["count"]) == forwards
        # the 3x first draw has been evicted: the window is below the all-time maximum
        assert all(w < a for w, a in zip(window[name], alltime[name])), (window, alltime)

    path = str(tmp_path / "scales.json")
    written = sf.save_scale_file(path, layers, margin=1.5)
    for name in names:
        want = oracle.static_amax(list(window[name]), 1.5)
        assert [written[name][t] for t in sf.TENSORS] == want, name

    loaded = sf.static_layers(path, DEV)
    q, k, v, cu = random_varlen(lens, H, seed=999, device=DEV)
    for name in names:
        A = tuple(written[name][t] for t in sf.TENSORS)
        out = loaded[name](q, k, v, _cu_dev(cu), cu)
        twin = fa.AttentionLayer(DEV, static_amax=window[name], margin=1.5)
        out2 = twin(q, k, v, _cu_dev(cu), cu)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), name
        s = fa.read_state(loaded[name].state)
        assert int(s["count"]) == 0                     # static: nothing observed
        for t in range(3):
            assert float(s["amax"][t]) == A[t]
            assert (float(s["scale"][t]), float(s["inv_scale"][t])) == oracle.scale_pair(A[t])
        sc = [oracle.scale_pair(a) for a in A]
        mx, mn = compare(bf16_to_f64(out), oracle_fp8_rows(q, k, v, cu, sc, SM))
        say(f"  {name}: A = {A}; fp8 vs oracle max-abs {mx:.3e} mean-abs {mn:.3e}")
        assert mx <= 1.5e-2 and mn <= 2e-3
