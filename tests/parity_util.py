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
# P is quantised relative to the running maximum over blocks of this many keys
# (FP8ATTN_KV_BLOCK in include/fp8attn.h); the oracle follows the same rule.
KV_BLOCK = 64


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


def oracle_fp8_rows(q, k, v, cu, scales_qkv, sm_scale, tokens=None, kv_block=KV_BLOCK):
    """Oracle FP8 attention on the given bf16 tensors (GPU or CPU) for `tokens` rows.

    scales_qkv: [(scale, inv)] * 3 as computed by the oracle. kv_block=None selects the
    global-row-maximum reading instead of the online-softmax rule.
    """
    luts = [quant_lut(s[1]) for s in scales_qkv]
    qb, kb, vb = bits(q), bits(k), bits(v)
    q8 = luts[0][qb] if tokens is None else None
    k8 = luts[1][kb]
    v8 = luts[2][vb]
    if tokens is None:
        return oracle.fp8_attention(q8, k8, v8, cu, scales_qkv[0][0], scales_qkv[1][0],
                                    scales_qkv[2][0], sm_scale, kv_block=kv_block)
    # only the requested query rows need quantising
    q8 = np.zeros(qb.shape, dtype=np.uint8)
    q8[tokens] = luts[0][qb[tokens]]
    return oracle.fp8_attention(q8, k8, v8, cu, scales_qkv[0][0], scales_qkv[1][0],
                                scales_qkv[2][0], sm_scale, tokens=tokens, kv_block=kv_block)


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


def hw_bound_rows(q8, k8, v8, cu, scales_qkv, sm_scale, tokens, kv_block=KV_BLOCK):
    """Per (row, head, channel) bound on |O_gpu - O_oracle| from the FP8 MFMA error.

    q8/k8/v8: E4M3 codes [T, H, d] (q8 needs only the requested rows). For row r the score
    of key j may be off by e_j = c * 2 * 2^-11 * max_c |q_c k_jc| (two 64-channel
    instructions); the running maximum by E = the largest e over the keys that hold a
    block maximum. As in the online rule, the weight of key j in block b is quantised
    relative to the running maximum m_b after that block, P~_j = exp(s_j - m_b) * 448, and
    enters the output scaled by exp(m_b - m_final). Each quantised weight then lies between
    the E4M3 codes of P~_j * exp(-+(e_j + 2E)), and the rescale factors within exp(+-2E);
    the PV and row-sum products add 2^-11 of their largest product per 64-key instruction;
    output rounding to bf16 adds 2^-9 |O|.
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
        nblk = (S + kv_block - 1) // kv_block
        for h in range(H):
            q = oracle.e4m3_decode(q8[rows, h])
            k = oracle.e4m3_decode(k8[lo:hi, h])
            v = oracle.e4m3_decode(v8[lo:hi, h]) * sv
            s = (q @ k.T) * c                                   # exact scores
            e = c * 2 * MFMA_REL_ERR * _max_products(q, k)
            E = np.zeros((len(rows), 1))
            for bb in range(nblk):
                j0, j1 = bb * kv_block, min(S, (bb + 1) * kv_block)
                am = np.argmax(s[:, j0:j1], axis=1) + j0
                E = np.maximum(E, e[np.arange(len(rows)), am][:, None])
            m_final = s.max(axis=1, keepdims=True)
            pt = np.zeros_like(s)                               # P~ against the running max
            w = np.zeros_like(s)                                # its factor exp(m_b - m_final)
            m_b = np.full((len(rows), 1), -np.inf)
            for bb in range(nblk):
                j0, j1 = bb * kv_block, min(S, (bb + 1) * kv_block)
                m_b = np.maximum(m_b, s[:, j0:j1].max(axis=1, keepdims=True))
                pt[:, j0:j1] = np.exp(s[:, j0:j1] - m_b) * oracle.E4M3_MAX
                w[:, j0:j1] = np.exp(m_b - m_final)
            lo8 = oracle.e4m3_decode(encode_nonneg(pt * np.exp(-(e + 2 * E)))) * w
            hi8 = oracle.e4m3_decode(encode_nonneg(pt * np.exp(e + 2 * E))) * w
            p = oracle.e4m3_decode(encode_nonneg(pt)) * w
            L = p.sum(axis=1, keepdims=True)
            O = (p @ v) / L
            dw = (hi8 - lo8) + p * (np.exp(2 * E) - 1.0)
            b = (dw @ np.abs(v) + dw.sum(axis=1, keepdims=True) * np.abs(O)) / L
            pv = np.zeros_like(O)
            ls = np.zeros((len(rows), 1))
            for bb in range(nblk):
                j0, j1 = bb * kv_block, min(S, (bb + 1) * kv_block)
                pv += (p[:, j0:j1, None] * np.abs(v[None, j0:j1, :])).max(axis=1)
                ls += p[:, j0:j1].max(axis=1, keepdims=True)
            b += MFMA_REL_ERR * (pv + ls * np.abs(O)) / L
            b += 2.0 ** -9 * np.abs(O)                           # bf16 output rounding
            out[dst, h] = b
    return out


def check_rows(got, want, bound, vstd, max_tol=MAX_ABS_TOL, mean_tol=MEAN_ABS_TOL):
    """Parity verdict in unit-variance units (errors divided by the V channel std).

    Every element must be within the stated max tolerance or within the hardware bound;
    the mean must meet the stated mean tolerance. Returns a dict of statistics.
    """
    err = np.abs(got - want) / vstd
    lim = np.maximum(max_tol, bound / vstd)
    bad = err > lim
    stats = {"max_abs_norm": float(err.max()), "mean_abs_norm": float(err.mean()),
             "max_abs": float(np.abs(got - want).max()),
             "n_over_stated": int((err > max_tol).sum()), "n_bad": int(bad.sum()),
             "n": int(err.size)}
    stats["ok"] = stats["n_bad"] == 0 and stats["mean_abs_norm"] <= mean_tol
    return stats


def v_channel_std(v: torch.Tensor) -> np.ndarray:
    """Empirical std of each (head, channel) of V over tokens, [H, d] (1 for unit variance)."""
    x = v.float()
    return x.reshape(-1, x.shape[1], x.shape[2]).std(dim=0).to("cpu").numpy().astype(np.float64)
