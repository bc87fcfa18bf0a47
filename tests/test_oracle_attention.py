"""Pins of the oracle's FP8 attention against closed forms, invariants and brute force.

* Q = 0 gives uniform weights, so O is the textbook mean of dec(v8) * scale_v;
* a single key gives O = dec(v8) * scale_v; a constant V comes out unchanged;
* a worked two-key case whose scores differ by ln 3: the max key gets p8 = 448 and the
  other E4M3(448/3) = 144, so O = (448 v1 + 144 v2) / 592 (normalising by the quantised
  weights; dividing by the unquantised sum would give 597.33 instead);
* weight rows sum to 1; permuting keys (with their values) changes nothing;
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
    # q . k1 = 8, q . k2 = 4 (raw dot products of E4M3 values); sigma chosen so the
    # score gap is ln 3: P~ = (1, 1/3), p8 = (448, E4M3(149.33) = 144).
    q8 = np.zeros((1, D), np.uint8)
    k8 = np.zeros((2, D), np.uint8)
    q8[0, 0] = e4m3_encode(np.array([2.0]))[0]
    k8[0, 0] = e4m3_encode(np.array([4.0]))[0]
    k8[1, 0] = e4m3_encode(np.array([2.0]))[0]
    v8 = np.zeros((2, D), np.uint8)
    v8[0, :] = e4m3_encode(np.array([1.0]))[0]
    v8[1, :] = e4m3_encode(np.array([-2.0]))[0]
    sigma = math.log(3.0) / 4.0
    out, p8, L = oracle.fp8_attention_head(q8, k8, v8, 1.0, 1.0, 1.0, sigma,
                                           return_weights=True)
    assert list(e4m3_decode(p8[0])) == [448.0, 144.0]
    assert L[0] == 592.0
    assert np.allclose(out[0], (448.0 * 1.0 + 144.0 * -2.0) / 592.0, rtol=1e-15)


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
    assert np.all(e4m3_decode(p8).max(axis=1) == 448.0)   # the row maximum maps to 448
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
            m = max(scores)
            p = []
            for s in scores:
                if s == -math.inf:
                    p.append(0.0)
                else:
                    p.append(float(e4m3_decode(e4m3_encode(np.array([math.exp(s - m) * 448.0])))[0]))
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


# ---------------------------------------------------------------- online-softmax rule
def test_online_single_block_equals_global():
    rng = np.random.default_rng(10)
    q8, k8, v8 = _codes(rng, (20, D), 2.0), _codes(rng, (50, D), 2.0), _codes(rng, (50, D))
    args = (0.02, 0.03, 0.004, 1 / math.sqrt(D))
    g = oracle.fp8_attention_head(q8, k8, v8, *args)
    for blk in (50, 64, 1000):
        assert np.array_equal(oracle.fp8_attention_head(q8, k8, v8, *args, kv_block=blk), g)


def test_online_equals_global_when_first_block_holds_max():
    rng = np.random.default_rng(11)
    q8, k8, v8 = _codes(rng, (1, D), 2.0), _codes(rng, (300, D), 2.0), _codes(rng, (300, D))
    raw = e4m3_decode(q8) @ e4m3_decode(k8).T
    first = int(np.argmax(raw[0]))
    perm = np.concatenate([[first], np.delete(np.arange(300), first)])
    k8, v8 = k8[perm], v8[perm]
    args = (0.02, 0.03, 0.004, 1 / math.sqrt(D))
    g = oracle.fp8_attention_head(q8, k8, v8, *args)
    for blk in (1, 7, 64):
        assert np.array_equal(oracle.fp8_attention_head(q8, k8, v8, *args, kv_block=blk), g)


def test_online_two_key_closed_form():
    # key 1 first with score s, key 2 next with s + ln 3, blocks of one key:
    # block 1: m = s, p8 = 448; block 2: rescale by 1/3, p8 = 448 ->
    # O = (448/3 v1 + 448 v2) / (448/3 + 448) = (v1 + 3 v2) / 4   (global rule: 0.27027)
    q8 = np.zeros((1, D), np.uint8)
    k8 = np.zeros((2, D), np.uint8)
    q8[0, 0] = e4m3_encode(np.array([2.0]))[0]
    k8[0, 0] = e4m3_encode(np.array([2.0]))[0]
    k8[1, 0] = e4m3_encode(np.array([4.0]))[0]
    v8 = np.zeros((2, D), np.uint8)
    v8[0, :] = e4m3_encode(np.array([1.0]))[0]
    v8[1, :] = e4m3_encode(np.array([-2.0]))[0]
    sigma = math.log(3.0) / 4.0
    out, w, L = oracle.fp8_attention_head(q8, k8, v8, 1.0, 1.0, 1.0, sigma, return_weights=True,
                                          kv_block=1)
    assert np.allclose(out[0], (1.0 + 3 * -2.0) / 4.0, rtol=1e-14)
    assert np.allclose(w[0], [0.25, 0.75], rtol=1e-14) and np.isclose(L[0], 448.0 * 4 / 3)
    out2 = oracle.fp8_attention_head(q8, k8, v8, 1.0, 1.0, 1.0, sigma, kv_block=2)
    assert np.allclose(out2[0], (448.0 * -2.0 + 144.0 * 1.0) / 592.0, rtol=1e-14)


def test_online_weights_sum_to_one_and_constant_v():
    rng = np.random.default_rng(12)
    q8, k8 = _codes(rng, (16, D), 3.0), _codes(rng, (333, D), 3.0)
    v8 = _codes(rng, (333, D))
    _, w, _ = oracle.fp8_attention_head(q8, k8, v8, 0.02, 0.03, 0.004, 1 / math.sqrt(D),
                                        return_weights=True, kv_block=64)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    vc = np.tile(v8[:1], (333, 1))
    out = oracle.fp8_attention_head(q8, k8, vc, 0.02, 0.03, 0.004, 1 / math.sqrt(D), kv_block=64)
    assert np.allclose(out, e4m3_decode(v8[:1]) * 0.004, rtol=1e-13, atol=0)


def _brute_force_online(q8, k8, v8, cu, sq, sk, sv, sigma, block):
    """Pure-Python loops: per row, blocks of keys of its own sequence, running maximum."""
    T, H, d = q8.shape
    dq, dk, dv = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    out = np.zeros((T, H, d))
    for i in range(len(cu) - 1):
        lo, hi = cu[i], cu[i + 1]
        for h in range(H):
            for r in range(lo, hi):
                m, L = -math.inf, 0.0
                acc = [0.0] * d
                for j0 in range(lo, hi, block):
                    js = list(range(j0, min(hi, j0 + block)))
                    sc = [sum(dq[r, h, c] * dk[j, h, c] for c in range(d)) * sq * sk * sigma
                          for j in js]
                    m_new = max([m] + sc)
                    a = math.exp(m - m_new) if m != -math.inf else 0.0
                    L *= a
                    acc = [x * a for x in acc]
                    for j, s in zip(js, sc):
                        p = float(e4m3_decode(e4m3_encode(np.array([math.exp(s - m_new) * 448.0])))[0])
                        L += p
                        for c in range(d):
                            acc[c] += p * dv[j, h, c]
                    m = m_new
                for c in range(d):
                    out[r, h, c] = acc[c] * sv / L
    return out


def test_online_brute_force_varlen():
    rng = np.random.default_rng(13)
    cu = [0, 9, 9, 23, 40]
    T, H, d = cu[-1], 2, 16
    q8, k8, v8 = _codes(rng, (T, H, d), 2.0), _codes(rng, (T, H, d), 2.0), _codes(rng, (T, H, d))
    args = (0.03, 0.02, 0.01, 0.3)
    got = oracle.fp8_attention(q8, k8, v8, cu, *args, kv_block=5)
    want = _brute_force_online(q8, k8, v8, cu, *args, block=5)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)
