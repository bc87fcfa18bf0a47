"""Pins of the oracle's FP8 attention against closed forms, invariants and brute force.

* Q = 0 gives uniform weights, so O is the textbook mean of dec(v8) * scale_v;
* a single key gives O = dec(v8) * scale_v; a constant V comes out unchanged;
* a worked two-key case with scores of 2.5 and 1.25 in log2 units: the reference
  exponent is 3, the weights E4M3(448 * 2^-0.5 = 316.8) = 320 and E4M3(448 * 2^-1.75 =
  133.2) = 128, so O = (320 v1 + 128 v2) / 448 (normalising by the quantised weights;
  dividing by the unquantised sum would give 450.0 instead; the exact maximum as the
  reference would give weights 448 and 192);
* weight rows sum to 1, the largest weight of a row is in [224, 448]; permuting keys
  (with their values) changes nothing;
* a single pass over 64-key blocks that takes each block's weights against the running
  reference exponent and rescales the partial sums by powers of two gives the same
  result (the property that lets a kernel find the maximum as it goes);
* packed varlen results equal separate per-sequence calls, which equal a dense
  block-diagonal-masked brute force written with pure-Python loops (T <= 64, H = 2);
* the float64 reference attention equals scipy's softmax-based formula (a library
  routine) and brute force;
* FP8 attention stays within cosine 0.998 of unquantised attention on unit-variance data.
  (E4M3 keeps 3 mantissa bits: its RMS relative rounding error is about 2.6 %, and Q, K, V
  and P are all rounded, so for flat attention the exact method's cosine is about
  1 - 0.052^2/2 = 0.9987; 0.999 is out of reach for any implementation on such data.)
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import e4m3_decode, e4m3_encode

D = 128


def _codes(rng, shape, scale=1.0):
    """Random E4M3 codes of N(0, scale^2) data quantised with a per-tensor dynamic scale."""
    x = rng.standard_normal(shape) * scale
    amax = float(np.max(np.abs(x)))
    _, inv = oracle.scale_pair(float(np.float32(amax)))
    return e4m3_encode(oracle.round_f32(x * inv))


def test_zero_query_gives_mean():
    rng = np.random.default_rng(0)
    S = 37
    q8 = np.zeros((5, D), np.uint8)
    k8 = _codes(rng, (S, D))
    v8 = _codes(rng, (S, D))
    sv = 0.0123
    out = oracle.fp8_attention_head(q8, k8, v8, 0.5, 0.25, sv, 1 / math.sqrt(D))
    want = e4m3_decode(v8).mean(axis=0) * sv
    assert np.allclose(out, want[None, :], rtol=1e-14, atol=0)


def test_single_key_and_constant_v():
    rng = np.random.default_rng(1)
    q8 = _codes(rng, (9, D))
    k8 = _codes(rng, (1, D))
    v8 = _codes(rng, (1, D))
    out = oracle.fp8_attention_head(q8, k8, v8, 0.1, 0.2, 0.3, 0.08)
    assert np.allclose(out, e4m3_decode(v8) * 0.3, rtol=1e-15, atol=0)
    S = 300
    k8 = _codes(rng, (S, D))
    v8 = np.tile(_codes(rng, (1, D)), (S, 1))
    out = oracle.fp8_attention_head(q8, k8, v8, 0.1, 0.2, 0.3, 0.08)
    assert np.allclose(out, e4m3_decode(v8[:1]) * 0.3, rtol=1e-14, atol=0)


def test_worked_two_key_example():
    # q . k1 = 8, q . k2 = 4 (raw dot products of E4M3 values); sigma = 0.3125 ln 2 puts
    # the scores at 2.5 and 1.25 in log2 units: M = 3, P~ = (2^-0.5, 2^-1.75),
    # p8 = (E4M3(316.78) = 320, E4M3(133.19) = 128).
    q8 = np.zeros((1, D), np.uint8)
    k8 = np.zeros((2, D), np.uint8)
    q8[0, 0] = e4m3_encode(np.array([2.0]))[0]
    k8[0, 0] = e4m3_encode(np.array([4.0]))[0]
    k8[1, 0] = e4m3_encode(np.array([2.0]))[0]
    v8 = np.zeros((2, D), np.uint8)
    v8[0, :] = e4m3_encode(np.array([1.0]))[0]
    v8[1, :] = e4m3_encode(np.array([-2.0]))[0]
    sigma = 0.3125 * math.log(2.0)
    out, p8, L = oracle.fp8_attention_head(q8, k8, v8, 1.0, 1.0, 1.0, sigma,
                                           return_weights=True)
    assert list(e4m3_decode(p8[0])) == [320.0, 128.0]
    assert L[0] == 448.0
    assert np.allclose(out[0], (320.0 * 1.0 + 128.0 * -2.0) / 448.0, rtol=1e-15)


def test_weights_sum_to_one_and_key_permutation():
    rng = np.random.default_rng(2)
    S = 200
    q8 = _codes(rng, (16, D), 3.0)
    k8 = _codes(rng, (S, D), 3.0)
    v8 = _codes(rng, (S, D))
    out, p8, L = oracle.fp8_attention_head(q8, k8, v8, 0.02, 0.03, 0.004, 1 / math.sqrt(D),
                                           return_weights=True)
    w = e4m3_decode(p8) / L[:, None]
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    top = e4m3_decode(p8).max(axis=1)           # the row maximum maps to 448 * (1/2, 1]
    assert np.all((top >= 224.0) & (top <= 448.0))
    assert len(set(top)) > 1                    # and not to one fixed code
    perm = rng.permutation(S)
    out2 = oracle.fp8_attention_head(q8, k8[perm], v8[perm], 0.02, 0.03, 0.004,
                                     1 / math.sqrt(D))
    assert np.array_equal(out, out2)


def _brute_force_dense(q8, k8, v8, cu, sq, sk, sv, sigma):
    """Dense T x T attention with -inf outside the diagonal blocks, pure Python loops."""
    T, H, d = q8.shape
    seq_of = [None] * T
    for i in range(len(cu) - 1):
        for t in range(cu[i], cu[i + 1]):
            seq_of[t] = i
    dq, dk, dv = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    out = np.zeros((T, H, d))
    for h in range(H):
        for r in range(T):
            scores = []
            for j in range(T):
                if seq_of[j] != seq_of[r]:
                    scores.append(-math.inf)
                    continue
                acc = 0.0
                for c in range(d):
                    acc += dq[r, h, c] * dk[j, h, c]
                scores.append(acc * sq * sk * sigma)
            M = math.ceil(max(scores) / math.log(2.0))
            p = []
            for s in scores:
                if s == -math.inf:
                    p.append(0.0)
                else:
                    x = 448.0 * 2.0 ** (s / math.log(2.0) - M)
                    p.append(float(e4m3_decode(e4m3_encode(np.array([x])))[0]))
            L = sum(p)
            for c in range(d):
                acc = 0.0
                for j in range(T):
                    acc += p[j] * dv[j, h, c]
                out[r, h, c] = acc * sv / L
    return out


def test_block_diagonal_isolation_brute_force():
    rng = np.random.default_rng(3)
    cu = [0, 7, 7, 20, 33]            # includes an empty sequence
    T, H, d = cu[-1], 2, 16
    q8 = _codes(rng, (T, H, d), 2.0)
    k8 = _codes(rng, (T, H, d), 2.0)
    v8 = _codes(rng, (T, H, d))
    args = (0.03, 0.02, 0.01, 0.3)
    packed = oracle.fp8_attention(q8, k8, v8, cu, *args)
    # separate per-sequence calls
    for i in range(len(cu) - 1):
        lo, hi = cu[i], cu[i + 1]
        if hi == lo:
            continue
        sep = oracle.fp8_attention(q8[lo:hi], k8[lo:hi], v8[lo:hi], [0, hi - lo], *args)
        assert np.array_equal(packed[lo:hi], sep)
    brute = _brute_force_dense(q8, k8, v8, cu, *args)
    assert np.allclose(packed, brute, rtol=1e-12, atol=1e-15)
    # row subsets give the same rows
    toks = [0, 6, 7, 19, 32]
    sub = oracle.fp8_attention(q8, k8, v8, cu, *args, tokens=toks)
    assert np.array_equal(sub, packed[toks])


def test_reference_attention_vs_library_and_brute_force():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((11, 8)), rng.standard_normal((11, 8))
    sigma = 0.37
    out = oracle.attention_f64(q, k, v, sigma)
    w = scipy.special.softmax(q @ k.T * sigma, axis=1)
    assert np.allclose(out, w @ v, rtol=1e-13, atol=1e-15)
    for r in range(5):
        e = [math.exp(sum(q[r, c] * k[j, c] for c in range(8)) * sigma) for j in range(11)]
        tot = sum(e)
        for c in range(8):
            assert abs(out[r, c] - sum(e[j] * v[j, c] for j in range(11)) / tot) < 1e-13


def test_fp8_close_to_unquantised():
    rng = np.random.default_rng(5)
    S, R = 512, 64
    x = [rng.standard_normal((n, D)) for n in (R, S, S)]
    bits = [(np.frombuffer(a.astype(np.float32).tobytes(), np.uint32) >> 16).astype(np.uint16)
            .reshape(a.shape) for a in x]
    vals = [oracle.bf16_bits_to_f64(b) for b in bits]
    sc = [oracle.scale_pair(oracle.amax_bf16(b)) for b in bits]
    codes = [oracle.quantize_bf16(b, s[1]) for b, s in zip(bits, sc)]
    sigma = float(np.float32(1 / math.sqrt(D)))
    o8 = oracle.fp8_attention_head(codes[0], codes[1], codes[2], sc[0][0], sc[1][0], sc[2][0], sigma)
    ref = oracle.attention_f64(vals[0], vals[1], vals[2], sigma)
    cos = np.sum(o8 * ref) / math.sqrt(np.sum(o8 * o8) * np.sum(ref * ref))
    assert 0.998 <= cos < 0.9995


def test_row_maximum_over_all_keys_not_a_prefix():
    # the reference is the row's own maximum over every key of its sequence: a row whose
    # largest score is its LAST key still has every weight quantised against that key's
    # exponent (computed here directly from the definition), whatever the number of keys
    # before it
    rng = np.random.default_rng(14)
    S = 300
    q8 = _codes(rng, (4, D), 2.0)
    k8 = _codes(rng, (S, D), 2.0)
    v8 = _codes(rng, (S, D))
    raw = e4m3_decode(q8) @ e4m3_decode(k8).T
    order = np.argsort(raw[0])                     # row 0: ascending scores, max key last
    k8, v8, raw = k8[order], v8[order], raw[:, order]
    args = (0.02, 0.03, 0.004, 1 / math.sqrt(D))
    out, p8, L = oracle.fp8_attention_head(q8, k8, v8, *args, return_weights=True)
    c = 0.02 * 0.03 / math.sqrt(D) / math.log(2.0)
    for r in range(4):
        M = math.ceil(max(raw[r]) * c)
        want = [e4m3_encode(np.array([448.0 * 2.0 ** (x * c - M)]))[0] for x in raw[r]]
        assert list(p8[r]) == want, r
    assert p8[0, -1] == p8[0].max() and e4m3_decode(p8[0, -1:])[0] >= 224.0


def _one_pass(q8, k8, v8, sq, sk, sv, sigma, block=64):
    """Blocks of keys in order, each block's weights E4M3(448 * 2^(t - M_run)) against the
    running reference exponent M_run = ceil(running max of t), the partial sums multiplied
    by 2^(M_old - M_new) whenever it grows (an independent evaluation of the rule)."""
    q, k, v = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    t_all = (q @ k.T) * (sq * sk * sigma / math.log(2.0))
    R = q.shape[0]
    M = np.full(R, -np.inf)
    acc = np.zeros((R, v.shape[1]))
    L = np.zeros(R)
    for j0 in range(0, k.shape[0], block):
        t = t_all[:, j0:j0 + block]
        Mn = np.maximum(M, np.ceil(t.max(axis=1)))
        f = np.where(np.isfinite(M), np.exp2(M - Mn), 0.0)   # exact powers of two
        acc *= f[:, None]
        L *= f
        p = e4m3_decode(e4m3_encode(448.0 * np.exp2(t - Mn[:, None])))
        acc += p @ v[j0:j0 + block]
        L += p.sum(axis=1)
        M = Mn
    return acc * sv / L[:, None]


def test_one_pass_with_power_of_two_rescale_gives_the_rule():
    # unit-variance rows keep every weight in E4M3's normal range, where the single pass
    # and the definition agree to float64 rounding, however the running maximum grows
    rng = np.random.default_rng(15)
    for S in (64, 200, 1000):
        q8 = _codes(rng, (32, D))
        k8 = _codes(rng, (S, D))
        v8 = _codes(rng, (S, D))
        args = (0.008, 0.008, 0.02, 1 / math.sqrt(D))
        want, p8, _ = oracle.fp8_attention_head(q8, k8, v8, *args, return_weights=True)
        assert e4m3_decode(p8).min() >= 2.0 ** -6        # the premise: no subnormal weight
        got = _one_pass(q8, k8, v8, *args)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-16), S
        t = e4m3_decode(q8) @ e4m3_decode(k8).T * (0.008 * 0.008 / math.sqrt(D) / math.log(2.0))
        if S > 64:   # the running reference did grow after the first block in some rows
            assert np.any(np.ceil(t[:, :64].max(axis=1)) < np.ceil(t.max(axis=1)))
        # with the exact maximum as the reference, the weights would differ
        s = t * math.log(2.0)
        exact_ref = e4m3_encode(448.0 * np.exp(s - s.max(axis=1, keepdims=True)))
        assert not np.array_equal(exact_ref, p8)
