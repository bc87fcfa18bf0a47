"""Random arguments through the C-ABI's host-side checks (CPU; no device is needed).

Thousands of seeded argument sets go through fp8attn_forward, fp8attn_quantize,
fp8attn_attend and fp8attn_workspace_bytes:
- sequence tables that start off zero, decrease, repeat, or reach the 32-bit limits;
- zero, negative and huge head counts, and head_dims other than 128;
- every flag combination, including invalid ones;
- NULL or fake addresses, with workspaces too small or huge;
- softmax scales that are NaN, infinite or non-positive.

Every call must return one of the documented codes. A negative code must come with a
message. A call that passes every check can only reach its first HIP call, which fails
without a device (FP8ATTN_EHIP), or return OK with nothing to launch (an empty batch).

The same test runs against a build whose host code is instrumented by AddressSanitizer:

    python -m fp8_dynamic_scaled_amd.build --asan
    ASAN_OPTIONS=detect_leaks=0 \\
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang --print-file-name=libclang_rt.asan-x86_64.so) \\
    FP8ATTN_TEST_LIB=fp8_dynamic_scaled_amd/lib/libfp8attn_asan.so \\
    python -m pytest tests/test_boundary_fuzz.py

(no report: the checks read only the host table entries they are given).
"""
import ctypes
import os
import random

import numpy as np
import pytest

from fp8_dynamic_scaled_amd import _lib

# Argument sets that pass every check go on to launch kernels on the fake addresses below,
# which only fails harmlessly where there is no GPU. Where the AMD GPU driver's device node
# exists, the test is skipped (checked without initialising HIP).
pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="launches on fake addresses: only without a GPU")

P, P2, NULL = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), ctypes.c_void_p(0)
CODES = {_lib.FP8ATTN_OK, _lib.FP8ATTN_EINVAL, _lib.FP8ATTN_EUNSUPPORTED, _lib.FP8ATTN_EHIP}


@pytest.fixture(scope="module")
def lib():
    path = os.environ.get("FP8ATTN_TEST_LIB")
    if not path:
        return _lib.load()
    h = ctypes.CDLL(path)
    for name, (res, args) in _lib.SIGNATURES.items():
        getattr(h, name).restype = res
        getattr(h, name).argtypes = args
    return h


STEPS = np.array([0, 1, 63, 64, 65, 1000, -5, 1 << 20, (1 << 31) - 1], dtype=np.int64)


def _table(rng, nrng, num_seqs):
    """A host cu_seqlens table of num_seqs + 1 entries (kept alive by the caller)."""
    first = 0 if rng.random() > 0.1 else rng.choice([1, -1])
    steps = STEPS[nrng.integers(0, len(STEPS), size=num_seqs)]
    vals = np.clip(first + np.concatenate([[0], np.cumsum(steps)]), -(1 << 31), (1 << 31) - 1)
    return np.ascontiguousarray(vals, dtype=np.int32)


def _check(lib, rc):
    assert rc in CODES, rc
    if rc != _lib.FP8ATTN_OK:
        assert lib.fp8attn_last_error()


def test_random_arguments_give_documented_codes(lib):
    rng = random.Random(20261203)
    nrng = np.random.default_rng(20261203)
    seen = set()
    for _ in range(4000):
        B = rng.choice([0, 1, 2, 3, 7, 64, 1 << 17, -1])
        table = _table(rng, nrng, B) if B >= 0 and rng.random() > 0.05 else None
        host = None if table is None else table.ctypes.data_as(_lib._i32p)
        H = rng.choice([0, 1, 2, 16, 40, -3, 1 << 20])
        D = rng.choice([128, 128, 64, 0, 256])
        flags = rng.choice([0, 1, 2, 3, 4])
        ws_bytes = rng.choice([0, 100, 1 << 30, 1 << 62])
        state, ws = rng.choice([P, NULL]), rng.choice([P2, NULL])
        sm = ctypes.c_float(rng.choice([0.0, -1.0, 0.1, float("nan"), float("inf")]))
        rc = lib.fp8attn_forward(state, P, P, P, P, host, B, H, D, sm, flags, ws, ws_bytes, P,
                                 NULL)
        _check(lib, rc)
        seen.add(rc)
        _check(lib, lib.fp8attn_quantize(state, P, P, P, P, host, B, H, D, ws, ws_bytes, NULL))
        _check(lib, lib.fp8attn_attend(state, P, host, B, H, D, sm, ws, ws_bytes, P, NULL))
        lib.fp8attn_workspace_bytes(rng.choice([0, 1, 1 << 40, -5]), B, H, D)
    # the sample reaches every kind of outcome
    assert {_lib.FP8ATTN_EINVAL, _lib.FP8ATTN_EUNSUPPORTED} <= seen
