"""Non-causal varlen attention with the FP8 P-quantisation rule (oracle; test only).

Sources:
  * vLLM-Omni "Quantized KV Cache", "Overview": FP8 flash attention for full-attention
    layers; Q/K/V quantised right before the operator. "Parameters": forwards listed by
    the step/layer selectors run in the native dtype instead.
  * Korean wiki "FP8 ViT 인코더 어텐션", "Requirements": the AMD backend is a varlen
    flash attention with per-tensor FP8 scales (packed sequences, cu_seqlens, no padding).
  * vLLM docs "FP8 ViT Encoder Attention", "Performance": head_dim 128.

The pages print no formula, so the attention is the textbook definition applied per
packed sequence (block-diagonal, non-causal), with these readings:
  * softmax scale sigma is an explicit argument (1/sqrt(d) by default);
  * scores use the dequantised E4M3 operands: s_j = (q8 . k8_j) * scale_q * scale_k * sigma;
  * P is quantised with a scale of 448 times a power of two: with m = max_j s_j, the row
    maximum over all keys of the row's sequence, and the reference exponent
    M = ceil(m * log2 e), P~_j = 2^(s_j log2 e - M) lies in (0, 1] (the largest weight in
    (1/2, 1]) and p8_j = E4M3(448 P~_j), so the largest code is in [224, 448];
  * the weights are the quantised p8_j normalised by their own sum (rows of weights sum
    to 1 and a constant V comes out unchanged); O is multiplied by scale_v.
The pages fix no scale for P. The reference is the row's own maximum, over every key (no
page fixes a block of keys, so how an implementation tiles them is not part of the
result), rounded up to a power of two: E4M3 rounding commutes with multiplication by a
power of two wherever both values are normal (>= 2^-6), so the weights of keys with
s_j log2 e <= M', taken against an integer reference exponent M' <= M and later
multiplied by 2^(M' - M), are these weights (away from that subnormal range). A flash-attention pass that finds the maximum as it
visits the keys can therefore reach this result without a second pass over them; with
the exact maximum as the reference it could not. Any reference in [m, m + ln 2) keeps
the largest weight where E4M3 has its full 3-bit precision; this one is the power of two.
Exactness: E4M3 values are multiples of 2^-9 below 2^9, so every product is a multiple
of 2^-18 below 2^18; the d = 128 score sum stays below 2^43 units and the PV sum over
up to ~2^17 keys below 2^53 units -- both are exact in float64 whatever the summation
order, so numpy's matrix product is an exact evaluation of those sums.
Rows of a sequence are independent; they are evaluated in groups of rows only to bound
memory, which changes no arithmetic.
"""

import math

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from .numerics import bf16_bits_to_f64

_ROW_GROUP = 512
_LOG2E = 1.0 / math.log(2.0)


def fp8_attention_head(q8, k8, v8, scale_q, scale_k, scale_v, sm_scale,
                       return_weights=False):
    """One (sequence, head): q8 [R, d], k8 [S, d], v8 [S, d] E4M3 codes -> O [R, d].

    With return_weights=True also returns the p8 codes [R, S] and L [R].
    """
    q = e4m3_decode(q8)
    k = e4m3_decode(k8)
    v = e4m3_decode(v8)
    c = float(scale_q) * float(scale_k) * float(sm_scale)
    R = q.shape[0]
    S = k.shape[0]
    out = np.zeros((R, q.shape[1]), dtype=np.float64)
    if S == 0:
        return (out, np.zeros((R, 0), np.uint8), np.zeros(R)) if return_weights else out
    all_p8 = np.zeros((R, S), dtype=np.uint8) if return_weights else None
    all_L = np.zeros(R) if return_weights else None
    for r0 in range(0, R, _ROW_GROUP):
        r1 = min(R, r0 + _ROW_GROUP)
        raw = q[r0:r1] @ k.T                      # exact
        s = raw * c
        t = s * _LOG2E                            # scores in log2 units
        M = np.ceil(np.max(t, axis=1, keepdims=True))   # reference exponent of the row
        p_tilde = np.exp2(t - M)                  # in (0, 1], the largest in (1/2, 1]
        p8 = e4m3_encode(p_tilde * E4M3_MAX)
        p = e4m3_decode(p8)
        L = np.sum(p, axis=1)                     # exact (multiples of 2^-9, < 2^53 units)
        out[r0:r1] = (p @ v) * float(scale_v) / L[:, None]
        if return_weights:
            all_p8[r0:r1] = p8
            all_L[r0:r1] = L
    if return_weights:
        return out, all_p8, all_L
    return out


def attention_f64(q, k, v, sm_scale):
    """Plain softmax attention of one (sequence, head) in float64: softmax(q k^T s) v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R = q.shape[0]
    out = np.zeros((R, q.shape[1]), dtype=np.float64)
    if k.shape[0] == 0:
        return out
    for r0 in range(0, R, _ROW_GROUP):
        r1 = min(R, r0 + _ROW_GROUP)
        s = (q[r0:r1] @ k.T) * float(sm_scale)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        out[r0:r1] = (p @ v) / np.sum(p, axis=1, keepdims=True)
    return out


def varlen_rows(cu_seqlens, tokens=None):
    """Group requested global token rows by sequence: list of (seq, lo, hi, local_rows).

    tokens=None means every row. local_rows are indices relative to the sequence start.
    """
    cu = [int(c) for c in cu_seqlens]
    groups = []
    tok = None if tokens is None else np.asarray(tokens, dtype=np.int64)
    for i in range(len(cu) - 1):
        lo, hi = cu[i], cu[i + 1]
        if tok is None:
            local = np.arange(hi - lo, dtype=np.int64)
        else:
            sel = tok[(tok >= lo) & (tok < hi)]
            local = sel - lo
        if local.size:
            groups.append((i, lo, hi, local))
    return groups


def _gather(groups, tokens, T):
    """Map (seq-local rows) back to positions in the output array."""
    if tokens is None:
        return None
    pos = {int(t): n for n, t in enumerate(np.asarray(tokens, dtype=np.int64))}
    return pos


def fp8_attention(q8, k8, v8, cu_seqlens, scale_q, scale_k, scale_v, sm_scale,
                  tokens=None):
    """Packed varlen FP8 attention. q8/k8/v8: E4M3 codes [T, H, d].

    Returns O [len(tokens), H, d] (or [T, H, d] when tokens is None) in float64, each
    sequence attending only to its own keys.
    """
    q8 = np.asarray(q8)
    T, H, d = q8.shape
    groups = varlen_rows(cu_seqlens, tokens)
    n_out = T if tokens is None else len(tokens)
    out = np.zeros((n_out, H, d), dtype=np.float64)
    pos = _gather(groups, tokens, T)
    for (_, lo, hi, local) in groups:
        rows = lo + local
        dst = rows if pos is None else np.array([pos[int(r)] for r in rows])
        for h in range(H):
            out[dst, h] = fp8_attention_head(q8[rows, h], k8[lo:hi, h], v8[lo:hi, h],
                                             scale_q, scale_k, scale_v, sm_scale)
    return out


def bf16_reference_attention(q_bits, k_bits, v_bits, cu_seqlens, sm_scale, tokens=None):
    """Packed varlen float64 attention on bf16 inputs (uint16 bit patterns [T, H, d]).

    This is the native-dtype path of the skip selectors and the unquantised reference
    for the cosine check.
    """
    q_bits = np.asarray(q_bits)
    T, H, d = q_bits.shape
    groups = varlen_rows(cu_seqlens, tokens)
    n_out = T if tokens is None else len(tokens)
    out = np.zeros((n_out, H, d), dtype=np.float64)
    pos = _gather(groups, tokens, T)
    for (_, lo, hi, local) in groups:
        rows = lo + local
        dst = rows if pos is None else np.array([pos[int(r)] for r in rows])
        for h in range(H):
            q = bf16_bits_to_f64(q_bits[rows, h])
            k = bf16_bits_to_f64(k_bits[lo:hi, h])
            v = bf16_bits_to_f64(v_bits[lo:hi, h])
            out[dst, h] = attention_f64(q, k, v, sm_scale)
    return out
