"""Graph capture of a whole FP8 attention forward, dynamic scaling included.

vLLM docs "FP8 ViT Encoder Attention", "Notes": on the pages' path dynamic scaling cannot
run under a full graph. Here the ring lives in device memory and every step (observe,
scales, quantise, attend) is a kernel launch with no allocation, copy, memset or host
sync, so the forward can be captured once and replayed. The test captures one forward of
a layer, then replays it on fresh inputs copied into the captured buffers, with eager
work and synchronisations between replays, and checks every replay bit for bit (output
and the whole state, ring included) against an eager twin layer fed the same
inputs, and against the oracle: the state (ring slots, count, window maximum, scales)
bit-exactly along the oracle's ring trajectory, the output at the stated tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_dynamic_scaled_amd as fa
from workloads import random_varlen

from parity_util import (OVER_TOL_CAP, OVER_TOL_CAP_OUTLIERS, bits, bf16_to_f64, check_rows,
                         hw_bound_rows, oracle_fp8_rows, oracle_ref_rows, quant_lut,
                         v_channel_std)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("mode", ["dynamic", "static", "skip"])
def test_captured_forward_replays_bit_identically(mode):
    H, lens = 2, [300, 77, 129]
    q, k, v, cu = random_varlen(lens, H, seed=77, device=DEV, outliers=True)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
    static = (40.0, 35.0, 30.0) if mode == "static" else None
    skip = mode == "skip"
    layer_g = fa.AttentionLayer(DEV, static_amax=static)
    layer_e = fa.AttentionLayer(DEV, static_amax=static)

    # one eager forward of each (the graph layer on a side stream, as capture requires its
    # allocations -- the workspace -- to exist before capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer_g(q, k, v, cu_d, cu, skip=skip)
    torch.cuda.current_stream().wait_stream(side)
    layer_e(q, k, v, cu_d, cu, skip=skip)
    torch.cuda.synchronize()
    ring = oracle.AmaxRing()                  # the oracle's view of layer_g's state
    if mode == "dynamic":
        ring.update([oracle.amax_bf16(bits(t)) for t in (q, k, v)])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = layer_g(q, k, v, cu_d, cu, skip=skip)
    torch.cuda.synchronize()
    say(f"{mode}: captured one forward")

    for r in range(6):
        # unit-variance draws, with x20 outlier channels on odd replays: the window maximum
        # of the dynamic ring rises and falls back as the replays go on
        q2, k2, v2, _ = random_varlen(lens, H, seed=100 + r, device=DEV, outliers=(r % 2 == 1))
        q.copy_(q2)
        k.copy_(k2)
        v.copy_(v2)
        g.replay()
        want = layer_e(q, k, v, cu_d, cu, skip=skip)
        torch.cuda.synchronize()
        assert torch.equal(out_g, want), (mode, r)
        assert torch.equal(layer_g.state, layer_e.state), (mode, r)
        s = fa.read_state(layer_g.state)
        say(f"  replay {r}: output and state identical; count {int(s['count'])}, "
            f"A {[float(x) for x in s['amax']]}")
        if mode == "dynamic":
            assert int(s["count"]) == r + 2
        # against the oracle
        sm = fa.default_softmax_scale()
        if skip:
            st = check_rows(bf16_to_f64(out_g), oracle_ref_rows(q, k, v, cu, sm),
                            v_channel_std(v)[None])
        else:
            if mode == "dynamic":
                A = ring.update([oracle.amax_bf16(bits(t)) for t in (q, k, v)])
                assert np.array_equal(s["ring"].astype(np.float64), ring.slots), r
                assert int(s["count"]) == ring.count
            else:
                A = oracle.static_amax(static, fa.DEFAULT_MARGIN)
            sc = [oracle.scale_pair(a) for a in A]
            for t in range(3):
                assert float(s["amax"][t]) == A[t], (r, t)
                assert (float(s["scale"][t]), float(s["inv_scale"][t])) == sc[t], (r, t)
            luts = [quant_lut(x[1]) for x in sc]
            q8, k8, v8 = (lut[bits(x)] for lut, x in zip(luts, (q, k, v)))
            st = check_rows(bf16_to_f64(out_g), oracle_fp8_rows(q, k, v, cu, sc, sm),
                            v_channel_std(v)[None],
                            lambda sel: hw_bound_rows(q8, k8, v8, cu, sc, sm, sel),
                            cap=OVER_TOL_CAP_OUTLIERS if r % 2 == 1 else OVER_TOL_CAP)
        say(f"  replay {r} vs oracle: {st}")
        assert st["ok"], (mode, r, st)
