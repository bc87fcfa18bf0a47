"""CPU checks of parity_util.hw_bound_rows, the per-element bound that the GPU parity tests
allow on top of the stated tolerance for the FP8 matrix core's inexact accumulation.

The bound is checked against a simulation of the effect it models: the online-softmax
rule (blocks of 64 keys, E4M3 weights relative to the running maximum) evaluated on scores
that carry an error of at most e_j = c * 2 * 2^-11 * max_c |q_c k_jc| each. Random
perturbations and ones with every score at an end of its interval must all stay within
the bound, including a row where a weight of the first block lies on an E4M3 rounding
midpoint relative to that block's maximum while the row's maximum lies in a later block
(the configuration that a bound taken relative to the global maximum misses).
"""
import math

import numpy as np

import oracle
from parity_util import KV_BLOCK, MFMA_REL_ERR, _max_products, encode_nonneg, hw_bound_rows

SM = float(np.float32(1.0 / math.sqrt(128)))


def _online(s, v, kv_block=KV_BLOCK):
    """The online rule on given (perturbed) scores s [S] for one row: output [d]."""
    m, O, L = -np.inf, np.zeros(v.shape[1]), 0.0
    for j0 in range(0, len(s), kv_block):
        blk = s[j0:j0 + kv_block]
        mn = max(m, blk.max())
        a = math.exp(m - mn) if m > -np.inf else 0.0
        O, L, m = O * a, L * a, mn
        p = oracle.e4m3_decode(oracle.e4m3_encode(np.exp(blk - m) * oracle.E4M3_MAX))
        O = O + p @ v[j0:j0 + kv_block]
        L += p.sum()
    return O / L


def _row_case(rng, S, plant_midpoint):
    """E4M3 codes of one query row, S keys and values, with unit scales. plant_midpoint:
    draw until some weight of the first block lies within the score error of an E4M3
    rounding midpoint relative to that block's maximum, while the row's maximum lies in a
    later block and the same weight relative to it is NOT near a midpoint."""
    for _ in range(1000):
        q = oracle.e4m3_encode(rng.standard_normal(128))
        k = oracle.e4m3_encode(rng.standard_normal((S, 128)))
        v = oracle.e4m3_encode(rng.standard_normal((S, 128)))
        if not plant_midpoint:
            return q, k, v
        qd, kd = oracle.e4m3_decode(q), oracle.e4m3_decode(k)
        s = (kd @ qd) * SM
        e = SM * 2 * MFMA_REL_ERR * _max_products(qd[None], kd)[0]
        m0, mf = s[:KV_BLOCK].max(), s.max()
        if mf <= m0 + 0.05:
            continue
        x0 = np.exp(s[:KV_BLOCK] - m0) * oracle.E4M3_MAX
        xf = np.exp(s[:KV_BLOCK] - mf) * oracle.E4M3_MAX
        r = e[:KV_BLOCK]
        near0 = oracle.e4m3_encode(x0 * np.exp(-r)) != oracle.e4m3_encode(x0 * np.exp(r))
        nearf = oracle.e4m3_encode(xf * np.exp(-r)) != oracle.e4m3_encode(xf * np.exp(r))
        if np.any(near0 & ~nearf & (x0 > 16.0)):
            return q, k, v
    raise AssertionError("no row with a weight on a midpoint found")


def _check(q, k, v, rng, trials=40):
    S = k.shape[0]
    qd, kd, vd = (oracle.e4m3_decode(x) for x in (q, k, v))
    sc = [(1.0, 1.0)] * 3
    bound = hw_bound_rows(q.reshape(1, 1, 128), k.reshape(S, 1, 128), v.reshape(S, 1, 128),
                          [0, S], sc, SM, np.array([0]))[0, 0]
    s = (kd @ qd) * SM
    e = SM * 2 * MFMA_REL_ERR * _max_products(qd[None], kd)[0]
    exact = _online(s, vd)
    worst = 0.0
    for t in range(trials):
        if t % 2 == 0:
            delta = rng.uniform(-1.0, 1.0, S) * e
        else:
            delta = rng.choice([-1.0, 1.0], S) * e           # every score at its extreme
        got = _online(s + delta, vd)
        # the GPU rounds its output to bf16 once
        got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(got))
        over = np.abs(got - exact) - bound
        worst = max(worst, float(over.max()))
    return worst, bound


def test_bound_covers_perturbed_scores_random_rows():
    rng = np.random.default_rng(1)
    for S in (1, 7, 64, 65, 100, 200):
        q, k, v = _row_case(rng, S, plant_midpoint=False)
        worst, _ = _check(q, k, v, rng)
        assert worst <= 0.0, (S, worst)


def test_bound_covers_a_weight_on_a_rounding_midpoint():
    rng = np.random.default_rng(2)
    q, k, v = _row_case(rng, 103, plant_midpoint=True)
    worst, bound = _check(q, k, v, rng, trials=80)
    assert worst <= 0.0, worst
    # the planted flip is large: the bound must allow far more than bf16 rounding here
    assert bound.max() > 2e-3


def test_bound_is_small_without_matrix_core_error(monkeypatch):
    import parity_util
    monkeypatch.setattr(parity_util, "MFMA_REL_ERR", 0.0)
    rng = np.random.default_rng(3)
    q, k, v = _row_case(rng, 150, plant_midpoint=False)
    S = k.shape[0]
    b = parity_util.hw_bound_rows(q.reshape(1, 1, 128), k.reshape(S, 1, 128), v.reshape(S, 1, 128),
                                  [0, S], [(1.0, 1.0)] * 3, SM, np.array([0]))[0, 0]
    O = _online((oracle.e4m3_decode(k) @ oracle.e4m3_decode(q)) * SM, oracle.e4m3_decode(v))
    # only the bf16 output rounding remains (plus the rescale term, zero with E = 0)
    assert np.all(b <= 2.0 ** -9 * np.abs(O) * (1 + 1e-9) + 1e-300)


def test_fast_nonnegative_encoder_equals_the_oracle():
    rng = np.random.default_rng(4)
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        vals, mids,                                          # every code and every tie
        np.nextafter(mids, 0), np.nextafter(mids, np.inf),   # just around each tie
        [0.0, 448.0, 464.0, 465.0, 1e9, np.inf, 2.0 ** -10, 2.0 ** -11],
        np.exp(rng.uniform(-25, 7, 200000)),                 # weights exp(s - m) * 448
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
