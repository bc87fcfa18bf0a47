"""CPU checks of parity_util.hw_bound_rows, the per-element bound that the GPU parity tests
allow (for at most a capped fraction of elements) on top of the stated tolerance, for the
FP8 matrix core's inexact accumulation.

The bound is checked against a simulation of the effect it models: the method's rule (E4M3
weights 448 * 2^(s log2 e - M), M the row maximum's exponent rounded up) evaluated on
scores that each carry an error of at most e_j = c * 2 * 2^-11 * max_c |q_c k_jc|, the
reference then taken from those perturbed scores -- either over all keys at once, or as a
single pass over 64-key tiles does it: each tile's weights against the running reference,
the partial sums rescaled by powers of two when it grows. Random perturbations and ones
with every score at an end of its interval must all stay within the bound, including a
row where a large weight lies on an E4M3 rounding midpoint, so that the perturbation moves
it by a whole E4M3 step, and rows whose weights reach E4M3's subnormal range.
"""
import math

import numpy as np

import oracle
from parity_util import (MFMA_KEYS, MFMA_REL_ERR, _max_products, encode_nonneg, hw_bound_rows,
                         score_slack)

SM = float(np.float32(1.0 / math.sqrt(128)))


LN2 = math.log(2.0)


def _rule(s, v, block=None):
    """The method's weights on given (perturbed) scores s [S] for one row: output [d].
    block: evaluate as one pass over tiles of that many keys, each tile's weights against
    the running reference exponent, the partial sums rescaled by powers of two."""
    t = s / LN2
    if block is None:
        p = oracle.e4m3_decode(oracle.e4m3_encode(np.exp2(t - np.ceil(t.max())) * oracle.E4M3_MAX))
        return (p @ v) / p.sum()
    M, acc, L = -np.inf, np.zeros(v.shape[1]), 0.0
    for j0 in range(0, len(t), block):
        tt = t[j0:j0 + block]
        Mn = max(M, math.ceil(tt.max()))
        f = 2.0 ** (M - Mn) if M > -np.inf else 0.0
        acc, L = acc * f, L * f
        p = oracle.e4m3_decode(oracle.e4m3_encode(np.exp2(tt - Mn) * oracle.E4M3_MAX))
        acc, L, M = acc + p @ v[j0:j0 + block], L + p.sum(), Mn
    return acc / L


def _errors(qd, kd):
    s = (kd @ qd) * SM
    e = SM * 2 * MFMA_REL_ERR * _max_products(qd[None], kd)[0] + score_slack(s, s.max())
    return s, e


def _row_case(rng, S, plant_midpoint, kstd=1.0):
    """E4M3 codes of one query row, S keys and values, with unit scales. plant_midpoint:
    draw until some weight above 16 lies within its score error of an E4M3 rounding
    midpoint, so that a perturbation inside the error moves it across. kstd widens the
    score spread (large values put many weights in E4M3's subnormal range)."""
    for _ in range(2000):
        q = oracle.e4m3_encode(rng.standard_normal(128))
        k = oracle.e4m3_encode(rng.standard_normal((S, 128)) * kstd)
        v = oracle.e4m3_encode(rng.standard_normal((S, 128)))
        if not plant_midpoint:
            return q, k, v
        qd, kd = oracle.e4m3_decode(q), oracle.e4m3_decode(k)
        s, e = _errors(qd, kd)
        x = np.exp2(s / LN2 - np.ceil(s.max() / LN2)) * oracle.E4M3_MAX
        near = oracle.e4m3_encode(x * np.exp(-e)) != oracle.e4m3_encode(x * np.exp(e))
        if np.any(near & (x > 16.0)):
            return q, k, v
    raise AssertionError("no row with a weight on a midpoint found")


def _check(q, k, v, rng, trials=40):
    S = k.shape[0]
    qd, kd, vd = (oracle.e4m3_decode(x) for x in (q, k, v))
    sc = [(1.0, 1.0)] * 3
    bound = hw_bound_rows(q.reshape(1, 1, 128), k.reshape(S, 1, 128), v.reshape(S, 1, 128),
                          [0, S], sc, SM, np.array([0]))[0, 0]
    s, e = _errors(qd, kd)
    exact = _rule(s, vd)
    assert np.allclose(exact, oracle.fp8_attention_head(q[None], k, v, 1.0, 1.0, 1.0, SM)[0],
                       rtol=1e-12, atol=1e-300)
    worst, moved = -np.inf, 0
    for t in range(trials):
        if t % 2 == 0:
            delta = rng.uniform(-1.0, 1.0, S) * e
        else:
            delta = rng.choice([-1.0, 1.0], S) * e           # every score at its extreme
        # half of the trials as the single pass over 64-key tiles, in a random key order
        if t % 4 < 2:
            got = _rule(s + delta, vd)
        else:
            perm = rng.permutation(S)
            got = _rule((s + delta)[perm], vd[perm], block=64)
        moved = max(moved, int(np.sum(got != exact)))
        # the GPU rounds its output to bf16 once
        got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(got))
        over = np.abs(got - exact) - bound
        worst = max(worst, float(over.max()))
    return worst, bound, moved


def test_bound_covers_perturbed_scores_random_rows():
    rng = np.random.default_rng(1)
    for S in (1, 7, 64, 65, 100, 200):
        q, k, v = _row_case(rng, S, plant_midpoint=False)
        worst, _, _ = _check(q, k, v, rng)
        assert worst <= 0.0, (S, worst)


def test_bound_covers_rows_with_subnormal_weights():
    # wide score spreads: many weights below 2^-6, where the single pass's provisional
    # references round on a finer grid than the rule's
    rng = np.random.default_rng(6)
    for S in (100, 300, 700):
        q, k, v = _row_case(rng, S, plant_midpoint=False, kstd=4.0)
        qd, kd = oracle.e4m3_decode(q), oracle.e4m3_decode(k)
        s, _ = _errors(qd, kd)
        w = np.exp2(s / LN2 - np.ceil(s.max() / LN2)) * oracle.E4M3_MAX
        assert np.mean(w < 2.0 ** -6) > 0.2                 # the premise
        worst, _, _ = _check(q, k, v, rng)
        assert worst <= 0.0, (S, worst)


def test_bound_covers_a_weight_on_a_rounding_midpoint():
    rng = np.random.default_rng(2)
    q, k, v = _row_case(rng, 103, plant_midpoint=True)
    worst, bound, moved = _check(q, k, v, rng, trials=80)
    assert worst <= 0.0, worst
    assert moved > 0                      # the perturbations did flip the planted weight
    # the planted flip is large: the bound must allow far more than bf16 rounding here
    assert bound.max() > 2e-3


def test_bound_is_small_without_matrix_core_error(monkeypatch):
    import parity_util
    monkeypatch.setattr(parity_util, "MFMA_REL_ERR", 0.0)
    monkeypatch.setattr(parity_util, "score_slack", lambda s, m: 0.0 * s)
    rng = np.random.default_rng(3)
    q, k, v = _row_case(rng, 150, plant_midpoint=False)
    S = k.shape[0]
    b = parity_util.hw_bound_rows(q.reshape(1, 1, 128), k.reshape(S, 1, 128), v.reshape(S, 1, 128),
                                  [0, S], [(1.0, 1.0)] * 3, SM, np.array([0]))[0, 0]
    qd, kd, vd = (oracle.e4m3_decode(x) for x in (q, k, v))
    O = _rule((kd @ qd) * SM, vd)
    # only the bf16 output rounding and the fp32 accumulation over the key blocks remain
    # (unit-variance scores keep every weight in E4M3's normal range)
    t = (kd @ qd) * SM / LN2
    p = oracle.e4m3_decode(oracle.e4m3_encode(np.exp2(t - np.ceil(t.max())) * oracle.E4M3_MAX))
    assert p.min() >= 2.0 ** -5
    nblk = (S + MFMA_KEYS - 1) // MFMA_KEYS
    acc = nblk * 2.0 ** -24 * ((p @ np.abs(vd)) / p.sum() + np.abs(O))
    assert np.all(b <= (2.0 ** -8 * np.abs(O) + acc) * (1 + 2.0 ** -7) + 1e-300)


def test_fast_nonnegative_encoder_equals_the_oracle():
    rng = np.random.default_rng(4)
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        vals, mids,                                          # every code and every tie
        np.nextafter(mids, 0), np.nextafter(mids, np.inf),   # just around each tie
        [0.0, 448.0, 464.0, 465.0, 1e9, np.inf, 2.0 ** -10, 2.0 ** -11],
        np.exp(rng.uniform(-25, 7, 200000)),                 # weights up to 448
        rng.uniform(0, 500, 100000)])
    assert np.array_equal(encode_nonneg(x), oracle.e4m3_encode(x))


def test_max_products_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(4):
        out = 1 + 30 * (rng.random(128) < 0.03)
        q = oracle.e4m3_decode(oracle.e4m3_encode(rng.standard_normal((9, 128)) * out))
        k = oracle.e4m3_decode(oracle.e4m3_encode(rng.standard_normal((333, 128)) * 2))
        want = np.abs(q[:, None, :] * k[None, :, :]).max(axis=2)
        assert np.array_equal(_max_products(q, k), want)
