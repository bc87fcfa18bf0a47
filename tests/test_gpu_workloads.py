"""GPU parity on the five full-size workloads (shapes, seeds and value distributions of
workloads.WORKLOADS), in the launch configuration the benchmark times.

Bytes (amax, ring, scales, every E4M3 byte of Q8/K8/V8t) are compared bit-exactly on every
workload (for the 20-forward ring and the DiT schedule: at the checked forwards); attention is compared on sampled rows (first/last rows of
every sequence plus seeded random rows, each row exact over all of its keys), in
unit-variance units (error / std of the V channel) against the stated tolerance, with the
per-element FP8 matrix-core bound of parity_util.hw_bound_rows for a capped fraction of
elements.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_dynamic_scaled_amd as fa
from workloads import CALIBRATION_FORWARD, WORKLOADS, dit_schedule, make_qkv

from parity_util import (OVER_TOL_CAP, OVER_TOL_CAP_OUTLIERS, bits, bf16_to_f64, check_rows,
                         cosine, hw_bound_rows, amax_exact,
                         oracle_fp8_rows, oracle_ref_rows, quant_lut, sample_tokens,
                         v_channel_std)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SM = fa.default_softmax_scale()


def say(msg):
    print(msg, flush=True)


def _cu(w):
    return list(w.cu_seqlens), torch.tensor(list(w.cu_seqlens), dtype=torch.int32, device=DEV)


def _amax3(q, k, v):
    return [amax_exact(t) for t in (q, k, v)]


def _check_state(st, A, count=None, ring=None):
    s = fa.read_state(st)
    for t in range(3):
        sc, inv = oracle.scale_pair(A[t])
        assert float(s["amax"][t]) == A[t], (t, float(s["amax"][t]), A[t])
        assert float(s["scale"][t]) == sc and float(s["inv_scale"][t]) == inv, t
    if count is not None:
        assert int(s["count"]) == count
    if ring is not None:
        assert np.array_equal(s["ring"].astype(np.float64), ring.slots)


def _check_bytes(ws, q, k, v, cu, sc):
    """Every byte of the FP8 workspace against the oracle's quantiser (streamed)."""
    T, H, D = q.shape
    B = len(cu) - 1
    q8, k8, v8t = fa.split_workspace(ws, T, B, H, D)
    luts = [quant_lut(x[1]) for x in sc]
    step = max(1, (1 << 24) // (H * D))
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        assert np.array_equal(q8[t0:t1].to("cpu").numpy(), luts[0][bits(q[t0:t1])]), ("q", t0)
        assert np.array_equal(k8[t0:t1].to("cpu").numpy(), luts[1][bits(k[t0:t1])]), ("k", t0)
    for i in range(B):
        lo, hi = cu[i], cu[i + 1]
        ps = fa.pad_start(lo, i)
        for h in range(H):
            got = v8t[h, :, ps:ps + hi - lo].to("cpu").numpy()
            want = luts[2][bits(v[lo:hi, h])].T
            assert np.array_equal(got, want), ("v", i, h)


def _fp8_parity(tag, out, q, k, v, cu, sc, toks, unit_variance=False, outliers=True):
    got = bf16_to_f64(out[torch.as_tensor(toks, device=DEV)])
    want = oracle_fp8_rows(q, k, v, cu, sc, SM, tokens=toks)
    vstd = 1.0 if unit_variance else v_channel_std(v)[None]
    luts = [quant_lut(x[1]) for x in sc]
    q8 = np.zeros(q.shape, np.uint8)
    q8[toks] = luts[0][bits(q[torch.as_tensor(toks, device=DEV)])]
    k8, v8 = luts[1][bits(k)], luts[2][bits(v)]
    st = check_rows(got, want, vstd,
                    lambda sel: hw_bound_rows(q8, k8, v8, cu, sc, SM, toks[np.asarray(sel)]),
                    cap=OVER_TOL_CAP_OUTLIERS if outliers else OVER_TOL_CAP)
    ref = oracle_ref_rows(q, k, v, cu, SM, tokens=toks)
    st["cos_gpu_vs_unquantised"] = cosine(got, ref)
    st["cos_oracle_vs_unquantised"] = cosine(want, ref)
    say(f"  {tag}: {st}")
    assert st["ok"], st
    assert st["cos_gpu_vs_unquantised"] >= st["cos_oracle_vs_unquantised"] - 1e-3
    return st


def _bf16_parity(tag, out, q, k, v, cu, toks):
    got = bf16_to_f64(out[torch.as_tensor(toks, device=DEV)])
    want = oracle_ref_rows(q, k, v, cu, SM, tokens=toks)
    st = check_rows(got, want, v_channel_std(v)[None])
    st["cos"] = cosine(got, want)
    say(f"  {tag}: {st}")
    assert st["ok"], st
    assert st["cos"] >= 0.9999


@pytest.mark.timeout(300)
def test_tiny_prefilled_ring_all_rows():
    w = WORKLOADS["tiny"]
    say(f"workload {w.name}: {w.description}")
    cu, cu_d = _cu(w)
    layer = fa.AttentionLayer(DEV)
    ring = oracle.AmaxRing()
    for f in range(w.prefill_forwards + 1):
        q, k, v = make_qkv(w, f, DEV)
        out = layer(q, k, v, cu_d, cu)
        A = ring.update(_amax3(q, k, v))
    torch.cuda.synchronize()
    _check_state(layer.state, A, count=4, ring=ring)
    sc = [oracle.scale_pair(a) for a in A]
    _check_bytes(layer._ws, q, k, v, cu, sc)
    toks = np.arange(w.total_tokens)
    _fp8_parity("tiny fp8, all rows", out, q, k, v, cu, sc, toks, unit_variance=True,
                outliers=False)
    skip = fa.forward(None, q, k, v, cu_d, cu, skip=True)
    _bf16_parity("tiny bf16, all rows", skip, q, k, v, cu, toks)


@pytest.mark.timeout(300)
def test_kernel_point_sampled_rows():
    w = WORKLOADS["kernel"]
    say(f"workload {w.name}: {w.description}")
    cu, cu_d = _cu(w)
    q, k, v = make_qkv(w, 0, DEV)
    layer = fa.AttentionLayer(DEV)
    out = layer(q, k, v, cu_d, cu)
    torch.cuda.synchronize()
    A = oracle.AmaxRing().update(_amax3(q, k, v))
    _check_state(layer.state, A, count=1)
    sc = [oracle.scale_pair(a) for a in A]
    _check_bytes(layer._ws, q, k, v, cu, sc)
    toks = sample_tokens(cu, 64, 128, seed=2)
    _fp8_parity("kernel fp8, sampled rows", out, q, k, v, cu, sc, toks)
    skip = fa.forward(None, q, k, v, cu_d, cu, skip=True)
    _bf16_parity("kernel bf16, sampled rows", skip, q, k, v, cu, toks)


@pytest.mark.timeout(300)
def test_qhd_static_scales_sampled_rows():
    w = WORKLOADS["qhd"]
    say(f"workload {w.name}: {w.description}")
    cu, cu_d = _cu(w)
    calib = _amax3(*make_qkv(w, CALIBRATION_FORWARD, DEV))
    torch.cuda.empty_cache()
    q, k, v = make_qkv(w, 0, DEV)
    layer = fa.AttentionLayer(DEV, static_amax=calib, margin=1.5)
    out = layer(q, k, v, cu_d, cu)
    torch.cuda.synchronize()
    A = oracle.static_amax(calib, 1.5)
    _check_state(layer.state, A, count=0)
    sc = [oracle.scale_pair(a) for a in A]
    _check_bytes(layer._ws, q, k, v, cu, sc)
    toks = sample_tokens(cu, 64, 128, seed=3)
    _fp8_parity("qhd fp8 static, sampled rows", out, q, k, v, cu, sc, toks)


@pytest.mark.timeout(900)
def test_4k_ring_over_20_forwards():
    w = WORKLOADS["4k"]
    say(f"workload {w.name}: {w.description}")
    cu, cu_d = _cu(w)
    layer = fa.AttentionLayer(DEV)
    ring = oracle.AmaxRing()
    toks = sample_tokens(cu, 64, 128, seed=4)
    for f in range(w.forwards):
        q, k, v = make_qkv(w, f, DEV)
        out = layer(q, k, v, cu_d, cu)
        A = ring.update(_amax3(q, k, v))
        _check_state(layer.state, A, count=f + 1, ring=ring)
        say(f"  forward {f}: ring state bit-exact (A = {A})")
        if f in (16, w.forwards - 1):           # right after the first eviction, and the last
            say(f"  forward {f}: window max {A}")
            sc = [oracle.scale_pair(a) for a in A]
            # every E4M3 byte of the one-pass dynamic quantisation (observe while quantising
            # with the other 15 slots, then re-quantise where the window maximum moved)
            _check_bytes(layer._ws, q, k, v, cu, sc)
            say(f"  forward {f}: every byte of Q8, K8, V8t bit-exact")
            _fp8_parity(f"4k fp8 forward {f}, sampled rows", out, q, k, v, cu, sc, toks,
                        outliers=w.outliers)
        del q, k, v, out
    assert ring.count == 20


@pytest.mark.timeout(1200)
def test_dit_steps_layers_skip_routing():
    w = WORKLOADS["dit"]
    say(f"workload {w.name}: {w.description}")
    cu, cu_d = _cu(w)
    steps, layers_sel = fa.parse_selector(w.skip_steps), fa.parse_selector(w.skip_layers)
    layers = [fa.AttentionLayer(DEV) for _ in range(w.layers)]
    rings = [oracle.AmaxRing() for _ in range(w.layers)]
    toks = sample_tokens(cu, 64, 128, seed=5)
    checked = set()
    for (f, step, layer, skip) in dit_schedule(w, steps, layers_sel):
        say(f"  forward {f}: step {step} layer {layer} {'bf16 (skip)' if skip else 'fp8'}")
        q, k, v = make_qkv(w, f, DEV)
        if skip:
            before = layers[layer].state.clone()
            out = fa.forward(None, q, k, v, cu_d, cu, skip=True)
            torch.cuda.synchronize()
            assert torch.equal(layers[layer].state, before)
            if (step, layer) == (0, 0):
                _bf16_parity("dit bf16 step 0 layer 0", out, q, k, v, cu, toks)
                checked.add("bf16")
        else:
            out = layers[layer](q, k, v, cu_d, cu)
            A = rings[layer].update(_amax3(q, k, v))
            _check_state(layers[layer].state, A, count=rings[layer].count, ring=rings[layer])
            if (step, layer) == (3, 7):
                sc = [oracle.scale_pair(a) for a in A]
                _check_bytes(layers[layer]._ws, q, k, v, cu, sc)
                say("  every byte of Q8, K8, V8t bit-exact")
                _fp8_parity("dit fp8 step 3 layer 7", out, q, k, v, cu, sc, toks)
                checked.add("fp8")
        del q, k, v, out
    counts = [int(fa.read_state(l.state)["count"]) for l in layers]
    say(f"  per-layer dynamic updates: {counts}")
    assert counts == [0, 0, 0, 2, 2, 2, 2, 2]
    assert checked == {"bf16", "fp8"}
