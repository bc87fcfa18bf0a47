"""GPU parity at the largest sizes.

Past 2^31 elements per tensor: 20 sequences of 56 000 tokens x 16 heads x 128
channels (2.29 G elements, 4.6 GB of bf16 per tensor), within the per-sequence 32-bit
limits of the C-ABI. Element offsets into Q, K, V, Q8, K8, V8t and the output then exceed
2^31, and every kernel must address them with 64-bit arithmetic.

Checked against the oracle: the amax (streamed through the host) and the ring/scales;
the E4M3 bytes of the last 1 000 tokens of Q8 and K8 and of the last sequence's V8t
columns for two heads; attention rows of the last sequence (sequences are independent, so
the oracle sees only that sequence). The one-pass dynamic path produces the state and the
workspace bytes checked here.

The longest single sequence the C-ABI accepts, FP8 and BF16 path (one sequence of one
tensor below 2^31 bytes): sampled attention rows over all of its keys.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_dynamic_scaled_amd as fa
from workloads import draw_tensor

from parity_util import (MAX_ABS_TOL, MEAN_ABS_TOL, amax_exact, bf16_to_f64, bits, compare,
                         cosine, oracle_fp8_rows, oracle_ref_rows, quant_lut)

# Over tens of thousands of keys the outputs of random inputs are small (about 1/sqrt of
# the key count), so the absolute tolerance alone would accept unrelated rows; the rows
# must also point the same way as the oracle's.
MIN_COSINE = 0.9999

pytestmark = pytest.mark.gpu
DEV = "cuda"
SM = fa.default_softmax_scale()
S, B, H = 56000, 20, 16


def say(msg):
    print(msg, flush=True)


@pytest.mark.timeout(600)
def test_tensors_past_2_pow_31_elements():
    T = S * B
    assert T * H * 128 > 2 ** 31
    say(f"large: {B} x {S} tokens, H={H}: {T * H * 128 / 1e9:.2f} G elements per tensor")
    q, k, v = (draw_tensor(T, H, 128, 9100 + t, DEV) for t in range(3))
    cu = [i * S for i in range(B + 1)]
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
    layer = fa.AttentionLayer(DEV)
    out = layer(q, k, v, cu_d, cu)
    torch.cuda.synchronize()
    say("  forward done; oracle amax (streamed)")

    A = oracle.AmaxRing().update([amax_exact(t) for t in (q, k, v)])
    s = fa.read_state(layer.state)
    sc = [oracle.scale_pair(a) for a in A]
    for t in range(3):
        assert float(s["amax"][t]) == A[t]
        assert float(s["scale"][t]) == sc[t][0] and float(s["inv_scale"][t]) == sc[t][1]

    # bytes at the far end of the workspace
    q8, k8, v8t = fa.split_workspace(layer._ws, T, B, H)
    luts = [quant_lut(x[1]) for x in sc]
    tail = slice(T - 1000, T)
    assert np.array_equal(q8[tail].to("cpu").numpy(), luts[0][bits(q[tail])])
    assert np.array_equal(k8[tail].to("cpu").numpy(), luts[1][bits(k[tail])])
    lo, hi = cu[-2], cu[-1]
    ps = fa.pad_start(lo, B - 1)
    for h in (0, H - 1):
        got = v8t[h, :, ps:ps + S].to("cpu").numpy()
        assert np.array_equal(got, luts[2][bits(v[lo:hi, h])].T), h
    say("  state and far-end bytes bit-exact")

    # attention rows of the last sequence
    rows = np.concatenate([np.arange(0, 48), np.arange(S - 48, S),
                           np.random.default_rng(7).integers(0, S, 32)])
    want = oracle_fp8_rows(q[lo:hi], k[lo:hi], v[lo:hi], [0, S], sc, SM, tokens=rows)
    got = bf16_to_f64(out[torch.as_tensor(lo + rows, device=DEV)])
    mx, mn = compare(got, want)
    cs = cosine(got, want)
    say(f"  last sequence, {len(rows)} rows: max-abs {mx:.3e} mean-abs {mn:.3e} "
        f"(|O| max {np.abs(want).max():.3e}), cosine {cs:.7f}")
    assert mx <= MAX_ABS_TOL and mn <= MEAN_ABS_TOL and cs >= MIN_COSINE


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", ["fp8", "bf16"])
def test_longest_sequence_at_the_32_bit_limit(path):
    # the C-ABI takes one sequence of a tensor (FP8 path: E4M3 bytes; BF16 path: bf16) up to
    # 2^31 - 1 bytes: the longest such sequence at 16 heads, through the full kernels
    h = 16
    bytes_per = 1 if path == "fp8" else 2
    s_max = ((1 << 31) - 1) // (h * 128 * bytes_per)
    say(f"longest {path} sequence: {s_max} tokens x {h} heads")
    q, k, v = (draw_tensor(s_max, h, 128, 9200 + t, DEV) for t in range(3))
    cu = [0, s_max]
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
    rows = np.concatenate([np.arange(0, 16), np.arange(s_max - 16, s_max),
                           np.random.default_rng(8).integers(0, s_max, 16)])
    if path == "fp8":
        layer = fa.AttentionLayer(DEV)
        out = layer(q, k, v, cu_d, cu)
        torch.cuda.synchronize()
        sc = [oracle.scale_pair(a) for a in oracle.AmaxRing().update([amax_exact(t) for t in (q, k, v)])]
        s = fa.read_state(layer.state)
        assert [float(x) for x in s["scale"]] == [x[0] for x in sc]
    else:
        out = fa.forward(None, q, k, v, cu_d, cu, skip=True)
        torch.cuda.synchronize()
    say("  kernels done; oracle rows head by head")
    want = np.zeros((len(rows), h, 128))
    for hh in range(h):            # one head at a time: bounded host memory, progress lines
        sl = slice(hh, hh + 1)
        if path == "fp8":
            want[:, sl] = oracle_fp8_rows(q[:, sl], k[:, sl], v[:, sl], cu, sc, SM, tokens=rows)
        else:
            want[:, sl] = oracle_ref_rows(q[:, sl], k[:, sl], v[:, sl], cu, SM, tokens=rows)
        say(f"    head {hh} done")
    got = bf16_to_f64(out[torch.as_tensor(rows, device=DEV)])
    mx, mn = compare(got, want)
    cs = cosine(got, want)
    say(f"  {len(rows)} rows over {s_max} keys: max-abs {mx:.3e} mean-abs {mn:.3e} "
        f"(|O| max {np.abs(want).max():.3e}), cosine {cs:.7f}")
    assert mx <= MAX_ABS_TOL and mn <= MEAN_ABS_TOL and cs >= MIN_COSINE
