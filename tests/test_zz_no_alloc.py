"""fp8attn_forward_noalloc through the C-ABI against fp8attn_forward.

The no-allocation entry point runs fp8attn_forward's kernels on the library's fixed
scratch array instead of a caller's workspace, so on the same inputs and the same state
its output (and, with FP8ATTN_OBSERVE, the state it writes) must equal fp8attn_forward's
bit for bit. Two calls in a row, the second on a smaller batch, show that what the first
call left in the scratch array does not leak into the second; the caller's workspace of
the reference call is filled with 0xFF beforehand for the same reason.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp8_dynamic_scaled_amd as fa
from fp8_dynamic_scaled_amd import _lib
from workloads import random_varlen

pytestmark = pytest.mark.gpu
DEV = "cuda"
SKIP, OBSERVE = 1, 2


def say(msg):
    print(msg, flush=True)


def _args(q, k, v, cu):
    host = np.asarray(cu, dtype=np.int32)
    cu_d = torch.tensor(host, dtype=torch.int32, device=DEV)
    return host, cu_d


def _call_ref(lib, st, q, k, v, cu, flags):
    host, cu_d = _args(q, k, v, cu)
    T, H, D = q.shape
    out = torch.empty_like(q)
    need = fa.workspace_bytes(T, len(cu) - 1, H, D)
    ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.fp8attn_forward(ctypes.c_void_p(0 if st is None else st.data_ptr()),
                             ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                             ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(cu_d.data_ptr()),
                             host.ctypes.data, len(cu) - 1, H, D, ctypes.c_float(0.0), flags,
                             ctypes.c_void_p(0 if flags & SKIP else ws.data_ptr()),
                             0 if flags & SKIP else ws.numel(), ctypes.c_void_p(out.data_ptr()),
                             stream)
    _lib.check("fp8attn_forward", rc)
    torch.cuda.synchronize()
    return out


def _call_noalloc(lib, st, q, k, v, cu, flags):
    host, cu_d = _args(q, k, v, cu)
    T, H, D = q.shape
    out = torch.empty_like(q)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.fp8attn_forward_noalloc(ctypes.c_void_p(0 if st is None else st.data_ptr()),
                                     ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                     ctypes.c_void_p(v.data_ptr()),
                                     ctypes.c_void_p(cu_d.data_ptr()), host.ctypes.data,
                                     len(cu) - 1, H, D, ctypes.c_float(0.0), flags,
                                     ctypes.c_void_p(out.data_ptr()), stream)
    _lib.check("fp8attn_forward_noalloc", rc)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_forward_two_calls_second_smaller():
    lib = _lib.load()
    big = random_varlen([1000, 37, 0, 300], 4, seed=401, device=DEV, outliers=True)
    small = random_varlen([200, 5], 2, seed=402, device=DEV)
    st_ref, st_na = fa.new_state(DEV), fa.new_state(DEV)
    torch.cuda.synchronize()
    for name, (q, k, v, cu) in (("big", big), ("small", small)):
        say(f"noalloc vs forward, dynamic (OBSERVE), {name}: lens {np.diff(cu).tolist()} "
            f"H={q.shape[1]}")
        o_ref = _call_ref(lib, st_ref, q, k, v, cu, OBSERVE)
        o_na = _call_noalloc(lib, st_na, q, k, v, cu, OBSERVE)
        assert torch.equal(o_ref, o_na), name
        assert torch.equal(st_ref, st_na), name
        # the state's scales as they now stand (no OBSERVE: the state is only read)
        say(f"noalloc vs forward, scales as set, {name}")
        o_ref = _call_ref(lib, st_ref, q, k, v, cu, 0)
        o_na = _call_noalloc(lib, st_na, q, k, v, cu, 0)
        assert torch.equal(o_ref, o_na), name
        say(f"noalloc vs forward, BF16 skip path, {name}")
        assert torch.equal(_call_ref(lib, None, q, k, v, cu, SKIP),
                           _call_noalloc(lib, None, q, k, v, cu, SKIP)), name
    assert int(fa.read_state(st_na)["count"]) == 2


def test_noalloc_rejects_a_batch_over_the_scratch_size():
    lib = _lib.load()
    T, H = 10881, 16
    assert fa.workspace_bytes(T, 1, H) > (64 << 20)
    q = torch.zeros((T, H, 128), dtype=torch.bfloat16, device=DEV)
    st = fa.new_state(DEV)
    torch.cuda.synchronize()
    with pytest.raises(_lib.Fp8AttnError) as ei:
        _call_noalloc(lib, st, q, q, q, [0, T], OBSERVE)
    assert ei.value.code == -1 and "fixed scratch" in str(ei.value)
    assert int(torch.count_nonzero(st)) == 0          # nothing ran on the state
