"""The one-pass dynamic forward (fp8attn_quantize_dynamic / FP8ATTN_OBSERVE) against the
separate observe + scales + quantise calls, bit for bit.

Both layers see the same inputs, forward after forward; after every forward the workspace
bytes (Q8, K8, V8t), the whole state and the attention output must be equal. The
sequence exercises: the first forward (empty ring, every tensor re-quantised), repeated
inputs (window maximum unchanged, no re-quantisation), a rising maximum on one tensor only,
falling draws that push the old maximum out of the 16-slot window, an all-zero tensor and
an empty batch (only the ring moves). Correctness against the oracle follows from the
separate path's own parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_dynamic_scaled_amd as fa
from workloads import random_varlen

from parity_util import amax_exact

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def _schedule():
    """(tag, seed, scale_q, scale_k, scale_v, lens) per forward."""
    lens = [300, 1, 77, 513, 0, 128, 64]
    out = [("first", 1, 1.0, 1.0, 1.0, lens), ("same", 1, 1.0, 1.0, 1.0, lens),
           ("same", 1, 1.0, 1.0, 1.0, lens), ("q up", 1, 2.0, 1.0, 1.0, lens),
           ("v up", 1, 2.0, 1.0, 3.0, lens), ("fresh", 2, 1.0, 1.0, 1.0, lens)]
    for f in range(14):                                    # evicts the raised maxima
        out.append((f"down {f}", 10 + f, 0.5, 0.6, 0.7, lens))
    out += [("zero v", 40, 0.5, 0.6, 0.0, lens), ("empty", 41, 1.0, 1.0, 1.0, [0, 0]),
            ("other shape", 42, 1.0, 1.0, 1.0, [2049, 31]), ("up again", 43, 4.0, 4.0, 4.0, [2049, 31])]
    return out


def test_one_pass_dynamic_equals_separate_calls():
    H = 2
    one = fa.AttentionLayer(DEV)                     # one_pass=True (the default)
    sep = fa.AttentionLayer(DEV, one_pass=False)
    ring = oracle.AmaxRing()
    for f, (tag, seed, sq, sk, sv, lens) in enumerate(_schedule()):
        q, k, v, cu = random_varlen(lens, H, seed=seed, device=DEV, outliers=True)
        q = (q.float() * sq).to(torch.bfloat16)
        k = (k.float() * sk).to(torch.bfloat16)
        v = (v.float() * sv).to(torch.bfloat16)
        cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
        o1 = one(q, k, v, cu_d, cu)
        o2 = sep(q, k, v, cu_d, cu)
        torch.cuda.synchronize()
        s1, s2 = fa.read_state(one.state), fa.read_state(sep.state)
        assert torch.equal(one.state, sep.state), (f, tag, s1, s2)
        # moved bit t: this forward's amax exceeds the 15 slots that stay (oracle ring)
        amax = [amax_exact(x) if x.numel() else 0.0 for x in (q, k, v)]
        slot = ring.count % oracle.RING_SLOTS
        rest = [float(np.max(np.delete(ring.slots[t], slot))) for t in range(3)]
        ring.update(amax)
        want = sum(1 << t for t in range(3) if amax[t] > rest[t])
        assert int(s1["moved"]) == want, (f, tag, int(s1["moved"]), want)
        T = q.shape[0]
        if T:
            B = len(cu) - 1
            for name, a, b in zip(("q8", "k8", "v8t"), fa.split_workspace(one._ws, T, B, H),
                                  fa.split_workspace(sep._ws, T, B, H)):
                assert torch.equal(a, b), (f, tag, name)
            assert torch.equal(o1, o2), (f, tag)
        say(f"  forward {f:2d} ({tag}): identical; count {int(s1['count'])}, "
            f"A {[float(x) for x in s1['amax']]}")


def test_forward_observe_flag_equals_layer_and_rejects_skip():
    H, lens = 3, [1000, 77]
    q, k, v, cu = random_varlen(lens, H, seed=8, device=DEV, outliers=True)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
    sep = fa.AttentionLayer(DEV, one_pass=False)
    st = fa.new_state(DEV)
    for _ in range(3):
        want = sep(q, k, v, cu_d, cu)
        got = fa.forward(st, q, k, v, cu_d, cu, observe=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert torch.equal(st, sep.state)
    with pytest.raises(ValueError):
        fa.forward(st, q, k, v, cu_d, cu, skip=True, observe=True)
