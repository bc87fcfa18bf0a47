"""Seeded synthetic workloads: shapes, seeds and bf16 input tensors.

This module holds only random-number generation and the workload shapes; none of the
method's arithmetic. Both the GPU path's tests/benchmark and the CPU oracle are fed from
it: the tensors are generated once (on the CPU or on the GPU with a seeded torch
generator) and the identical bf16 bytes are given to both sides.

The workloads stand in for the pages' real inputs, which are not available here:
  * Qwen3-VL ViT encoder images, 3 per request, at QHD and 4K (vLLM docs "FP8 ViT Encoder
    Attention", "Performance": end-to-end encoder table) -> packed varlen batches of
    3 images, 90x160 and 135x240 patches;
  * the core-kernel shape of the same section (head_dim 128, seq_len 8192);
  * Wan2.2-style DiT video full attention with step/layer skip selectors (vLLM-Omni
    "Quantized KV Cache", "Configuration" and "Parameters").
Values: z ~ N(0, 1) in fp32 times a per-element factor, rounded once to bf16 (RNE).
"Outliers": n_out = max(1, round(0.001 * H * d)) of the H*d hidden columns, chosen per
tensor from their own seed and fixed across forwards, are multiplied by 20.
Seeds: workload k (1..5) has base 1000*k; a draw uses 1000*k + 100*f + t (f = forward
index, f = 99 for the calibration draw, t = 0/1/2 for q/k/v); outlier columns use
1000*k + 7 + t.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                       # k in the seed formulas
    cu_seqlens: Tuple[int, ...]
    num_heads: int
    head_dim: int = HEAD_DIM
    outliers: bool = False           # 0.1 % of hidden columns scaled by 20
    per_head_std: bool = False       # per (forward, tensor, head) std ~ U[0.5, 2]
    scaling: str = "dynamic"         # "dynamic" ring or "static" calibrated amax x margin
    prefill_forwards: int = 0        # dynamic forwards observed before the tested one
    forwards: int = 1                # forwards in one run of the workload
    steps: int = 0                   # DiT: denoising steps (0 = not a DiT workload)
    layers: int = 0                  # DiT: transformer layers
    skip_steps: str = ""             # DiT: selector of steps kept in bf16
    skip_layers: str = ""            # DiT: selector of layers kept in bf16
    description: str = ""

    @property
    def total_tokens(self) -> int:
        return self.cu_seqlens[-1]

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def seq_lens(self) -> List[int]:
        c = self.cu_seqlens
        return [c[i + 1] - c[i] for i in range(len(c) - 1)]

    def flops(self) -> float:
        """4 * sum_i S_i^2 * d * H: the QK^T and PV products of a block-diagonal forward."""
        return 4.0 * sum(s * s for s in self.seq_lens) * self.head_dim * self.num_heads

    def elements(self) -> int:
        """Elements per tensor, T * H * d."""
        return self.total_tokens * self.num_heads * self.head_dim


WORKLOADS = {
    "tiny": Workload("tiny", 1, (0, 256), 2, prefill_forwards=3,
                     description="1 sequence of 256, H=2, N(0,1); ring pre-filled by 3 "
                                 "forwards; dynamic scaling"),
    "kernel": Workload("kernel", 2, (0, 8192), 16, outliers=True,
                       description="1 sequence of 8192, H=16, N(0,1) with x20 outlier "
                                   "columns; dynamic scaling"),
    "qhd": Workload("qhd", 3, (0, 14400, 28800, 43200), 16, outliers=True, scaling="static",
                    description="3 QHD images of 90x160 patches, H=16, N(0,1)+outliers; "
                                "static scales = calibration amax x 1.5"),
    "4k": Workload("4k", 4, (0, 32400, 64800, 97200), 16, per_head_std=True, forwards=20,
                   description="3 4K images of 135x240 patches, H=16, per-head std "
                               "U[0.5,2]; 20 forwards through one ring"),
    "dit": Workload("dit", 5, (0, 57600), 40, outliers=True, forwards=32, steps=4, layers=8,
                    skip_steps="0,1", skip_layers="0-2",
                    description="16 frames x 45x80 patches = 57600 tokens, H=40, "
                                "N(0,1)+outliers; 4 steps x 8 layers, skip steps 0,1 and "
                                "layers 0-2 to bf16"),
}

CALIBRATION_FORWARD = 99


def draw_seed(w: Workload, forward: int, tensor: int) -> int:
    return 1000 * w.index + 100 * forward + tensor


def outlier_seed(w: Workload, tensor: int) -> int:
    return 1000 * w.index + 7 + tensor


def _generator(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_columns(w: Workload, tensor: int) -> torch.Tensor:
    """Indices (into the H*d hidden) of the outlier columns of one tensor (CPU tensor)."""
    hidden = w.num_heads * w.head_dim
    n_out = max(1, round(0.001 * hidden))
    g = _generator("cpu", outlier_seed(w, tensor))
    return torch.randperm(hidden, generator=g)[:n_out]


def draw_tensor(T: int, H: int, d: int, seed: int, device="cpu", outlier_cols=None,
                per_head_std=False) -> torch.Tensor:
    """One bf16 [T, H, d] tensor: z ~ N(0,1) fp32 times factors, rounded once to bf16."""
    g = _generator(device, seed)
    factor = torch.ones(H * d, dtype=torch.float32, device=device)
    if per_head_std:
        std = torch.empty(H, dtype=torch.float32, device=device).uniform_(0.5, 2.0,
                                                                          generator=g)
        factor = factor * std.repeat_interleave(d)
    if outlier_cols is not None and len(outlier_cols) > 0:
        factor[outlier_cols.to(device)] *= 20.0
    z = torch.randn((T, H * d), dtype=torch.float32, device=device, generator=g)
    z.mul_(factor)
    return z.to(torch.bfloat16).view(T, H, d)


def make_qkv(w: Workload, forward: int, device="cpu"):
    """(q, k, v) bf16 [T, H, d] for one forward of a workload."""
    out = []
    for t in range(3):
        cols = outlier_columns(w, t) if w.outliers else None
        out.append(draw_tensor(w.total_tokens, w.num_heads, w.head_dim,
                               draw_seed(w, forward, t), device, cols, w.per_head_std))
    return tuple(out)


def cu_seqlens_tensor(cu, device="cpu") -> torch.Tensor:
    return torch.tensor(list(cu), dtype=torch.int32, device=device)


def random_varlen(seq_lens, num_heads, seed, device="cpu", head_dim=HEAD_DIM,
                  outliers=False, scale=1.0):
    """Seeded (q, k, v, cu_seqlens) for an arbitrary list of sequence lengths.

    Used by parity tests to span several tiles, ragged tails and empty sequences.
    """
    cu = [0]
    for s in seq_lens:
        cu.append(cu[-1] + int(s))
    T = cu[-1]
    hidden = num_heads * head_dim
    qkv = []
    for t in range(3):
        cols = None
        if outliers:
            g = _generator("cpu", seed * 10 + 7 + t)
            cols = torch.randperm(hidden, generator=g)[:max(1, round(0.001 * hidden))]
        x = draw_tensor(T, num_heads, head_dim, seed * 10 + t, device, cols)
        if scale != 1.0:
            x = (x.float() * scale).to(torch.bfloat16)
        qkv.append(x)
    return qkv[0], qkv[1], qkv[2], cu


def dit_schedule(w: Workload, skip_steps, skip_layers):
    """List of (forward, step, layer, skip) for a DiT workload, in execution order."""
    sched = []
    for step in range(w.steps):
        for layer in range(w.layers):
            f = step * w.layers + layer
            sched.append((f, step, layer, (step in skip_steps) or (layer in skip_layers)))
    return sched
