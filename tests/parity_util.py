"""Helpers shared by the GPU parity tests and the benchmark's checks.

The oracle always starts from the same bf16 bytes the GPU saw (copied to the host) and
computes its own amax, scales and E4M3 codes; nothing the HIP path produced is fed to it.
"""
import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

MAX_ABS_TOL = 1.5e-2     # attention output vs the oracle, unit-variance inputs
MEAN_ABS_TOL = 2e-3
# At most a fraction of the compared elements may exceed MAX_ABS_TOL, and each of those only
# within its hardware bound (hw_bound_rows): the matrix core's accumulation error can move a
# single E4M3 weight across a rounding midpoint, which on a short row moves the output by
# more than the stated tolerance; the cap keeps the bound from absorbing any number of such
# elements. Every weight, the largest included (448 times a power of two, not 448 itself),
# sits on the E4M3 grid wherever the score puts it, so any of them can be moved. The error
# is relative to the largest product of a score, so it, and the number of moved weights,
# grow with outlier channels and with the softmax scale:
#   unit-variance inputs at the default scale (the regime the stated tolerance is for):
#   1e-4 (measured: at most 5.8e-5, on a batch of rows of 1 to 513 keys);
#   inputs with x20 outlier channels, or a softmax scale 3.4 x the default: 5e-3
#   (measured: at most 1.8e-3).
OVER_TOL_CAP = 1e-4
OVER_TOL_CAP_OUTLIERS = 5e-3
# keys per FP8 MFMA of the PV and row-sum products (the K dimension of one instruction):
# the hardware bound groups their accumulation error by these blocks
MFMA_KEYS = 64


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).to("cpu").numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits(t))


def amax_exact(t: torch.Tensor) -> float:
    """Oracle amax of a (possibly large) bf16 tensor, streamed in chunks to the host."""
    flat = t.detach().reshape(-1)
    best = 0.0
    step = 1 << 27
    for s in range(0, flat.numel(), step):
        best = max(best, oracle.amax_bf16_bits(bits(flat[s:s + step])))
    return best


def quant_lut(inv: float) -> np.ndarray:
    """Oracle E4M3 code of every bf16 pattern under multiplier inv (a 65536-entry table:
    quantisation is a function of the bf16 value alone, so gathering from this table is
    exactly oracle.quantize_bf16 applied element by element)."""
    return oracle.quantize_bf16(np.arange(65536, dtype=np.uint32).astype(np.uint16), inv)


def sample_tokens(cu, per_seq_edge=64, per_seq_random=128, seed=0):
    """First/last rows of every sequence plus seeded random rows (global token ids)."""
    rng = np.random.default_rng(seed)
    toks = []
    for i in range(len(cu) - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi == lo:
            continue
        s = set(range(lo, min(hi, lo + per_seq_edge))) | set(range(max(lo, hi - per_seq_edge), hi))
        if hi - lo > 2 * per_seq_edge:
            s |= set(int(x) for x in rng.integers(lo, hi, size=per_seq_random))
        toks.extend(sorted(s))
    return np.array(sorted(set(toks)), dtype=np.int64)


def oracle_fp8_rows(q, k, v, cu, scales_qkv, sm_scale, tokens=None):
    """Oracle FP8 attention on the given bf16 tensors (GPU or CPU) for `tokens` rows.

    scales_qkv: [(scale, inv)] * 3 as computed by the oracle.
    """
    luts = [quant_lut(s[1]) for s in scales_qkv]
    qb, kb, vb = bits(q), bits(k), bits(v)
    q8 = luts[0][qb] if tokens is None else None
    k8 = luts[1][kb]
    v8 = luts[2][vb]
    if tokens is None:
        return oracle.fp8_attention(q8, k8, v8, cu, scales_qkv[0][0], scales_qkv[1][0],
                                    scales_qkv[2][0], sm_scale)
    # only the requested query rows need quantising
    q8 = np.zeros(qb.shape, dtype=np.uint8)
    q8[tokens] = luts[0][qb[tokens]]
    return oracle.fp8_attention(q8, k8, v8, cu, scales_qkv[0][0], scales_qkv[1][0],
                                scales_qkv[2][0], sm_scale, tokens=tokens)


def oracle_ref_rows(q, k, v, cu, sm_scale, tokens=None):
    return oracle.bf16_reference_attention(bits(q), bits(k), bits(v), cu, sm_scale, tokens)


def compare(gpu_rows: np.ndarray, want: np.ndarray):
    d = np.abs(gpu_rows - want)
    return float(d.max()), float(d.mean())


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.reshape(-1)
    b = b.reshape(-1)
    return float(np.dot(a, b) / math.sqrt(np.dot(a, a) * np.dot(b, b)))


# ---------------------------------------------------------------------------------
# Hardware accumulation bound of the FP8 matrix core.
# gfx950's v_mfma_f32_32x32x64_f8f6f4 does not sum its 64 products exactly: measured on
# random E4M3 operands with outlier channels, the error of one instruction stays below
# 2^-11 of the largest |product| in it (probe over 256 x 64 x 32 dot products, worst
# 2^-11.1 for a two-instruction d = 128 sum). The attention parity therefore allows, on
# top of the stated tolerance, the output change those score/PV/row-sum errors can cause.
MFMA_REL_ERR = 2.0 ** -11          # per instruction, relative to its largest |product|
_LOG2E = 1.0 / math.log(2.0)


_NONNEG_VALUES = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0x00..0x7E
_NONNEG_MIDS = (_NONNEG_VALUES[:-1] + _NONNEG_VALUES[1:]) / 2


def encode_nonneg(a):
    """E4M3 codes of non-negative values (RNE, saturating), by binary search over the 126
    midpoints between consecutive codes: a value on a midpoint takes the even code, which
    is the even mantissa (the low code bit is the low mantissa bit, and across a binade
    edge the larger value has mantissa 0). Equal to oracle.e4m3_encode on a >= 0
    (tests/test_hw_bound.py); used where the bound encodes millions of weights."""
    a = np.asarray(a, dtype=np.float64)
    i = np.searchsorted(_NONNEG_MIDS, a, side="left")
    on_mid = (i < len(_NONNEG_MIDS)) & (a == _NONNEG_MIDS[np.minimum(i, len(_NONNEG_MIDS) - 1)])
    i = np.where(on_mid & (i % 2 == 1), i + 1, i)
    return i.astype(np.uint8)


def _max_products(q, k):
    """max_c |q[r,c] k[j,c]| for every (row, key), exactly: the inputs are E4M3 values, so
    each product is exact in float32 (at most 8 significant bits, below 2^18), and so is
    their maximum. One pass per channel over a [rows, keys] buffer."""
    qa = np.abs(np.asarray(q, dtype=np.float64)).astype(np.float32).T.copy()   # [d, rows]
    ka = np.abs(np.asarray(k, dtype=np.float64)).astype(np.float32).T.copy()   # [d, keys]
    out = np.zeros((qa.shape[1], ka.shape[1]), dtype=np.float32)
    tmp = np.empty_like(out)
    for c in range(qa.shape[0]):
        np.multiply(qa[c][:, None], ka[c][None, :], out=tmp)
        np.maximum(out, tmp, out=out)
    return out.astype(np.float64)


def score_slack(s, m):
    """Bound on the fp32 evaluation error of 448 * 2^(s log2 e - M) in the kernel, in
    natural-log units: the softmax constant c = scale_q * scale_k * sigma * log2 e is a few
    binary32 roundings, M - log2 448 one more, the exponent s * c - (M - log2 448) is one
    FMA, and v_exp_f32 is within 1 ulp; with M < m log2 e + 1, 2^-21 (16 + |m| + |s - m|)
    covers them all."""
    return 2.0 ** -21 * (16.0 + np.abs(m) + np.abs(s - m))


def hw_bound_rows(q8, k8, v8, cu, scales_qkv, sm_scale, tokens):
    """Per (row, head, channel) bound on |O_gpu - O_oracle| from the FP8 MFMA error.

    q8/k8/v8: E4M3 codes [T, H, d] (q8 needs only the requested rows). For row r the score
    of key j may be off by e_j = c * 2 * 2^-11 * max_c |q_c k_jc| (two 64-channel
    instructions) plus score_slack. The kernel's reference exponent, taken from its own
    scores (and, before the last key tile, from the running maximum), differs from the
    oracle's M only by whole powers of two, which scale every weight and the row sum alike
    and so leave O unchanged -- except where a weight falls below E4M3's normal range
    (2^-6) on one of the grids, where the two roundings differ by at most 2^-9 at the
    oracle's scale (the kernel's grid is at most twice as coarse, 2^-8 apart). So each
    weight lies between the E4M3 codes of 448 * 2^(s_j log2 e - M) * exp(-+e_j), widened by
    2^-9 on each side when the upper value is below 2^-5; that moves O by at most
    sum_j width_j (|v_j| + |O|) / L_lo (L_lo: the row sum of the lower ends); the PV and
    row-sum MFMAs add 2^-11 of their largest product per 64-key instruction, fp32
    accumulation over the key blocks 2^-24 per block (the power-of-two rescales of the
    partial sums are exact), and the output's rounding to bf16 2^-8 of its value.
    """
    sq, sk, sv = scales_qkv[0][0], scales_qkv[1][0], scales_qkv[2][0]
    c = sq * sk * sm_scale
    T, H, d = q8.shape
    out = np.zeros((len(tokens), H, d))
    pos = {int(t): n for n, t in enumerate(tokens)}
    for (i, lo, hi, local) in oracle.varlen_rows(cu, tokens):
        rows = lo + local
        dst = np.array([pos[int(r)] for r in rows])
        S = hi - lo
        nblk = (S + MFMA_KEYS - 1) // MFMA_KEYS
        for h in range(H):
            q = oracle.e4m3_decode(q8[rows, h])
            k = oracle.e4m3_decode(k8[lo:hi, h])
            v = oracle.e4m3_decode(v8[lo:hi, h]) * sv
            s = (q @ k.T) * c                                   # exact scores
            m = s.max(axis=1, keepdims=True)
            e = c * 2 * MFMA_REL_ERR * _max_products(q, k) + score_slack(s, m)
            t = s * _LOG2E
            M = np.ceil(t.max(axis=1, keepdims=True))
            pt = np.exp2(t - M) * oracle.E4M3_MAX
            sub = np.where(pt * np.exp(e) < 2.0 ** -5, 2.0 ** -9, 0.0)
            lo8 = np.maximum(oracle.e4m3_decode(encode_nonneg(pt * np.exp(-e))) - sub, 0.0)
            hi8 = oracle.e4m3_decode(encode_nonneg(pt * np.exp(e))) + sub
            p = oracle.e4m3_decode(encode_nonneg(pt))
            L = p.sum(axis=1, keepdims=True)
            L_lo = lo8.sum(axis=1, keepdims=True)
            O = (p @ v) / L
            dw = hi8 - lo8
            b = (dw @ np.abs(v) + dw.sum(axis=1, keepdims=True) * np.abs(O)) / L_lo
            pv = np.zeros_like(O)
            ls = np.zeros((len(rows), 1))
            for bb in range(nblk):
                j0, j1 = bb * MFMA_KEYS, min(S, (bb + 1) * MFMA_KEYS)
                pv += (hi8[:, j0:j1, None] * np.abs(v[None, j0:j1, :])).max(axis=1)
                ls += hi8[:, j0:j1].max(axis=1, keepdims=True)
            b += MFMA_REL_ERR * (pv + ls * np.abs(O)) / L_lo
            b += nblk * 2.0 ** -24 * ((hi8 @ np.abs(v)) / L_lo + np.abs(O))
            # the output is rounded to bf16 once (8 significant bits: at most 2^-8 of the
            # value it rounds, which is within b of O)
            b += 2.0 ** -8 * (np.abs(O) + b) * (1 + 2.0 ** -20)
            out[dst, h] = b
    return out


def check_rows(got, want, vstd, bound_fn=None, max_tol=MAX_ABS_TOL, mean_tol=MEAN_ABS_TOL,
               cap=OVER_TOL_CAP):
    """Parity verdict in unit-variance units (errors divided by vstd, the V channel std:
    1.0 for unit-variance inputs). got/want: [rows, H, d].

    Every element must be within the stated max tolerance, except at most a fraction `cap`
    of them, each within its hardware bound; the mean must meet the stated mean tolerance.
    bound_fn(sel) returns hw_bound_rows for the rows `sel` (indices into got's first axis);
    it is evaluated only for rows that hold an element over the stated tolerance. Without
    it no element may exceed the tolerance. Returns a dict of statistics.
    """
    err = np.abs(got - want) / vstd
    over = err > max_tol
    n = int(err.size)
    sel = np.nonzero(over.reshape(over.shape[0], -1).any(axis=1))[0]
    n_over = int(over.sum())
    if sel.size == 0:
        n_bad, worst_ratio = 0, 0.0
    elif bound_fn is None:
        n_bad, worst_ratio = n_over, float("inf")
    else:
        lim = bound_fn(sel) / vstd
        e_sel = err[sel]
        bad = over[sel] & (e_sel > lim)
        n_bad = int(bad.sum())
        worst_ratio = float((e_sel[over[sel]] / lim[over[sel]]).max())
    stats = {"max_abs_norm": float(err.max()), "mean_abs_norm": float(err.mean()),
             "max_abs": float(np.abs(got - want).max()),
             "n_over_stated": n_over, "frac_over_stated": n_over / max(n, 1),
             "n_over_bound": n_bad, "worst_over_stated_err_per_bound": worst_ratio, "n": n}
    stats["ok"] = (n_bad == 0 and stats["mean_abs_norm"] <= mean_tol and n_over <= cap * n)
    return stats


def v_channel_std(v: torch.Tensor) -> np.ndarray:
    """Empirical std of each (head, channel) of V over tokens, [H, d] (1 for unit variance)."""
    x = v.float()
    return x.reshape(-1, x.shape[1], x.shape[2]).std(dim=0).to("cpu").numpy().astype(np.float64)
