"""Step/layer skip selectors (host logic).

vLLM-Omni user guide "Quantized KV Cache", section "Parameters": the denoising-step and
transformer-layer selectors are strings of comma-separated integers and inclusive ranges
(examples there: "0,1,4-6" for steps, "0-2,10" for layers); listed steps or layers keep
attention in the native dtype, every other eligible full-attention forward takes the FP8
path. Section "Configuration" shows "0,1" and "0-2".

Readings where the page is silent: whitespace around items is ignored; None or "" selects
nothing; indices are 0-based non-negative integers; a range a-b needs a <= b; anything
else is an error rather than being ignored.
"""
from typing import Iterable, Optional, Set


def parse_selector(spec: Optional[str]) -> Set[int]:
    """Parse "0,1,4-6" -> {0, 1, 4, 5, 6}. Raises ValueError on malformed input."""
    if spec is None:
        return set()
    text = str(spec).strip()
    if not text:
        return set()
    out: Set[int] = set()
    for raw in text.split(","):
        item = raw.strip()
        if not item:
            raise ValueError(f"empty item in selector {spec!r}")
        if "-" in item:
            lo_s, sep, hi_s = item.partition("-")
            lo_s, hi_s = lo_s.strip(), hi_s.strip()
            if not (lo_s.isdigit() and hi_s.isdigit()):
                raise ValueError(f"bad range {item!r} in selector {spec!r}")
            lo, hi = int(lo_s), int(hi_s)
            if lo > hi:
                raise ValueError(f"descending range {item!r} in selector {spec!r}")
            out.update(range(lo, hi + 1))
        else:
            if not item.isdigit():
                raise ValueError(f"bad index {item!r} in selector {spec!r}")
            out.add(int(item))
    return out


def skip_fp8(step: int, layer: int, skip_steps: Iterable[int], skip_layers: Iterable[int]) -> bool:
    """True when this (step, layer) forward stays in the native dtype."""
    return step in set(skip_steps) or layer in set(skip_layers)
