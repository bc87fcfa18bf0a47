"""Online per-tensor FP8 (E4M3) attention for AMD Instinct MI355X (gfx950).

Per attention call: observe the Q/K/V amax, update a 16-slot amax ring (or use a static
calibrated amax times a margin), quantise Q/K/V to E4M3 and run a non-causal varlen
flash-attention forward on FP8 matrix cores; or, for forwards selected by the step/layer
skip selectors, the same attention in BF16. All of it runs in hand-written HIP kernels
behind the C-ABI of include/fp8attn.h; this package is a thin ctypes binding over it.
"""
from .api import (AttentionLayer, DEFAULT_MARGIN, HEAD_DIM, attend, default_softmax_scale, forward,
                  new_state, observe_amax, pad_start, quantize, quantize_dynamic, read_state, scales,
                  split_workspace, state_bytes, state_reset, workspace_bytes)
from ._lib import Fp8AttnError, LIB_PATH, load as load_library
from .selectors import parse_selector, skip_fp8
from . import scale_file
from .scale_file import load_scale_file, save_scale_file, static_layers

__all__ = [
    "AttentionLayer", "DEFAULT_MARGIN", "HEAD_DIM", "attend", "default_softmax_scale", "forward",
    "new_state", "observe_amax", "pad_start", "quantize", "quantize_dynamic", "read_state", "scales",
    "split_workspace", "state_bytes", "state_reset", "workspace_bytes", "Fp8AttnError",
    "LIB_PATH", "load_library", "parse_selector", "skip_fp8",
    "scale_file", "load_scale_file", "save_scale_file", "static_layers",
]
