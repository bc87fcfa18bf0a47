"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fp8attn.h declares, and rejects bad arguments on the host before enqueuing
anything (no HIP call happens on these paths, so they run without a device)."""
import ctypes
import os
import re

import numpy as np
import pytest

import fp8_dynamic_scaled_amd as fa
from fp8_dynamic_scaled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8attn.h")

# fake, 256-byte aligned device addresses: validation must fail before touching them
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    pat = r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fp8attn_[a-z_]+)\s*\("
    return sorted(set(re.findall(pat, text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 11, names
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert set(_lib.SIGNATURES) == set(names)


def test_sizes(lib):
    assert lib.fp8attn_state_bytes() == 1280
    from fp8_dynamic_scaled_amd.api import STATE_DTYPE
    assert STATE_DTYPE.itemsize == 1280
    assert STATE_DTYPE.fields["cur"][1] % 64 == 0     # each stripe a 64-byte line
    T, B, H, D = 43200, 3, 16, 128
    Tp = (T + 127) // 128 * 128 + 128 * B
    assert lib.fp8attn_workspace_bytes(T, B, H, D) == 2 * T * H * D + H * D * Tp
    assert lib.fp8attn_workspace_bytes(-1, 1, 16, 128) == 0
    assert lib.fp8attn_workspace_bytes(10, 0, 16, 128) == 0
    assert lib.fp8attn_workspace_bytes(10, 1, 0, 128) == 0


def _cu(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr


def _fwd(lib, **kw):
    a = dict(state=P, q=P, k=P, v=P, cu=P, cu_host=_cu([0, 8, 16]), num_seqs=2, H=2, D=128,
             sm=0.0, flags=0, ws=P2, ws_bytes=1 << 30, out=P, stream=NULL)
    a.update(kw)
    return lib.fp8attn_forward(a["state"], a["q"], a["k"], a["v"], a["cu"], a["cu_host"],
                               a["num_seqs"], a["H"], a["D"], ctypes.c_float(a["sm"]),
                               a["flags"], a["ws"], a["ws_bytes"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=NULL), -1, "non-NULL"),
    (dict(cu=NULL), -1, "cu_seqlens"),
    (dict(cu_host=None), -1, "cu_seqlens"),
    (dict(num_seqs=0), -1, "num_seqs"),
    (dict(H=0), -1, "num_heads"),
    (dict(D=64), -2, "head_dim"),
    (dict(cu_host=_cu([1, 8, 16])), -1, "cu_seqlens[0]"),
    (dict(cu_host=_cu([0, 8, 4])), -1, "decreases"),
    (dict(flags=4), -1, "flag"),
    (dict(flags=3), -1, "exclude each other"),
    (dict(ws_bytes=100), -1, "workspace"),
    (dict(ws=NULL), -1, "workspace"),
    (dict(state=NULL), -1, "state"),
    (dict(out=NULL), -1, "out"),
    (dict(q=ctypes.c_void_p(0x10008)), -1, "aligned"),
    (dict(sm=float("nan")), -1, "softmax_scale"),
    (dict(cu_host=_cu([0, 1 << 30, (1 << 31) - 1]), H=2), -1, "exceeds"),
    # 32-bit offsets inside the attention kernels: one sequence of one tensor ...
    (dict(cu_host=_cu([0, 1 << 20, (1 << 20) + 8]), H=16), -2, "longest sequence"),
    # ... and one head's V8t rows (2^17 sequences of 128 tokens: padded keys 3 * 2^24)
    (dict(cu_host=_cu(list(range(0, (1 << 24) + 1, 128))), num_seqs=1 << 17, H=1), -2,
     "padded tokens"),
])
def test_forward_rejects(lib, kw, code, needle):
    assert _fwd(lib, **kw) == code
    assert needle in lib.fp8attn_last_error().decode()


def test_skip_path_rejects_sequences_beyond_32bit_byte_offsets(lib):
    # 2^19 tokens x 16 heads x 128 channels x 2 bytes = 2^31: fine for FP8, not for BF16
    cu = _cu([0, 1 << 19])
    assert _fwd(lib, state=NULL, ws=NULL, ws_bytes=0, flags=1, cu_host=cu, num_seqs=1, H=16) == -2
    assert "BF16" in lib.fp8attn_last_error().decode()


def test_skip_path_needs_no_state_or_workspace_but_checks_the_rest(lib):
    # on the skip path a NULL state/workspace is fine; a bad head_dim still fails first
    assert _fwd(lib, state=NULL, ws=NULL, ws_bytes=0, flags=1, D=96) == -2


def test_quantize_rejects(lib):
    rc = lib.fp8attn_quantize(NULL, P, P, P, P, _cu([0, 4]), 1, 1, 128, P2, 1 << 20, NULL)
    assert rc == -1 and "state" in lib.fp8attn_last_error().decode()
    rc = lib.fp8attn_quantize(P, P, P, P, P, _cu([0, 4]), 1, 1, 128, P2, 10, NULL)
    assert rc == -1 and "workspace" in lib.fp8attn_last_error().decode()


def test_scales_and_observe_reject(lib):
    f3 = (ctypes.c_float * 3)
    assert lib.fp8attn_scales(NULL, 0, None, ctypes.c_float(1.5), NULL) == -1
    assert lib.fp8attn_scales(P, 7, None, ctypes.c_float(1.5), NULL) == -1
    assert "mode" in lib.fp8attn_last_error().decode()
    assert lib.fp8attn_scales(P, 1, None, ctypes.c_float(1.5), NULL) == -1
    assert lib.fp8attn_scales(P, 1, f3(1.0, -2.0, 3.0), ctypes.c_float(1.5), NULL) == -1
    # amax and margin each finite, their binary32 product not: rejected before any launch
    assert lib.fp8attn_scales(P, 1, f3(1.0, 3.0e38, 3.0), ctypes.c_float(1.5), NULL) == -1
    assert "overflows" in lib.fp8attn_last_error().decode()
    assert lib.fp8attn_scales(P, 1, f3(1.0, float("inf"), 3.0), ctypes.c_float(1.5), NULL) == -1
    assert lib.fp8attn_scales(P, 1, f3(1.0, 2.0, 3.0), ctypes.c_float(0.0), NULL) == -1
    assert lib.fp8attn_scales(P, 1, f3(1.0, 2.0, 3.0), ctypes.c_float(float("nan")), NULL) == -1
    assert "margin" in lib.fp8attn_last_error().decode()
    assert lib.fp8attn_observe_amax(NULL, P, P, P, 128, NULL) == -1
    assert lib.fp8attn_observe_amax(P, P, P, P, -1, NULL) == -1
    assert lib.fp8attn_observe_amax(P, NULL, P, P, 128, NULL) == -1
    assert lib.fp8attn_observe_amax(P, ctypes.c_void_p(0x10002), P, P, 128, NULL) == -1
    assert lib.fp8attn_state_reset(NULL, NULL) == -1


def test_quantize_dynamic_rejects(lib):
    rc = lib.fp8attn_quantize_dynamic(NULL, P, P, P, P, _cu([0, 4]), 1, 1, 128, P2, 1 << 20, NULL)
    assert rc == -1 and "state" in lib.fp8attn_last_error().decode()
    rc = lib.fp8attn_quantize_dynamic(P, P, P, P, P, _cu([0, 4]), 1, 1, 128, P2, 10, NULL)
    assert rc == -1 and "workspace" in lib.fp8attn_last_error().decode()
    rc = lib.fp8attn_quantize_dynamic(P, P, P, P, P, _cu([0, 4]), 1, 1, 96, P2, 1 << 20, NULL)
    assert rc == -2 and "head_dim" in lib.fp8attn_last_error().decode()


def test_flag_constants_agree():
    import fp8_dynamic_scaled_amd._lib as L
    hdr = open(HEADER).read()
    for name in ("FP8ATTN_SKIP", "FP8ATTN_OBSERVE", "FP8ATTN_DYNAMIC", "FP8ATTN_STATIC"):
        m = re.search(rf"#define {name} (\d+)u?", hdr)
        assert m and int(m.group(1)) == getattr(L, name), name


def test_attend_rejects(lib):
    args = dict(state=P, cu=P, cu_host=_cu([0, 8]), B=1, H=2, D=128, ws=P2, wsb=1 << 30, out=P)
    def call(**kw):
        a = dict(args); a.update(kw)
        return lib.fp8attn_attend(a["state"], a["cu"], a["cu_host"], a["B"], a["H"], a["D"],
                                  ctypes.c_float(0.0), a["ws"], a["wsb"], a["out"], NULL)
    assert call(ws=NULL) == -1 and "workspace" in lib.fp8attn_last_error().decode()
    assert call(state=NULL) == -1 and "state" in lib.fp8attn_last_error().decode()
    assert call(D=256) == -2
    assert call(wsb=64) == -1
    assert call(out=NULL) == -1
    assert call(cu_host=_cu([0, -3])) == -1


def test_errors_raise_in_binding():
    with pytest.raises(_lib.Fp8AttnError) as ei:
        _lib.check("fp8attn_forward", _fwd(_lib.load(), D=64))
    assert ei.value.code == -2


def test_pad_start_regions_hold_their_sequences():
    rng = np.random.default_rng(0)
    for _ in range(200):
        lens = rng.integers(0, 400, size=rng.integers(1, 8))
        cu = np.concatenate([[0], np.cumsum(lens)])
        starts = [fa.pad_start(int(cu[i]), i) for i in range(len(lens) + 1)]
        Tp = (int(cu[-1]) + 127) // 128 * 128 + 128 * len(lens)
        assert starts[-1] == Tp
        for i, s in enumerate(lens):
            assert starts[i] % 128 == 0
            # the next sequence starts at or past the end of the last whole 128-column tile
            # that holds this one: tiles of 64 or 128 keys read past its end see only zeros
            assert starts[i + 1] - starts[i] >= (int(s) + 127) // 128 * 128


def test_binding_rejects_host_tensors_before_any_gpu_call():
    # the Python binding refuses host memory (and non-tensors) for every device argument,
    # before the library sees an address
    import torch
    q = torch.zeros(8, 2, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.forward(None, q, q, q, cu, [0, 8], skip=True)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.quantize(torch.zeros(1280, dtype=torch.uint8), q, q, q, cu, [0, 8])
    with pytest.raises(TypeError, match="torch.Tensor"):
        fa.observe_amax(None, q, q, q)
    with pytest.raises(TypeError, match="torch.Tensor"):
        fa.scales(None, "dynamic")


def _fwd_noalloc(lib, **kw):
    a = dict(state=P, q=P, k=P, v=P, cu=P, cu_host=_cu([0, 8, 16]), num_seqs=2, H=2, D=128,
             sm=0.0, flags=0, out=P, stream=NULL)
    a.update(kw)
    return lib.fp8attn_forward_noalloc(a["state"], a["q"], a["k"], a["v"], a["cu"],
                                       a["cu_host"], a["num_seqs"], a["H"], a["D"],
                                       ctypes.c_float(a["sm"]), a["flags"], a["out"],
                                       a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=NULL), -1, "non-NULL"),
    (dict(cu_host=None), -1, "cu_seqlens"),
    (dict(D=64), -2, "head_dim"),
    (dict(flags=3), -1, "exclude each other"),
    (dict(state=NULL), -1, "state"),
    (dict(out=NULL), -1, "out"),
    # one sequence of 10 881 tokens x 16 heads needs more workspace than the fixed scratch
    # (10 880 fill it exactly)
    (dict(cu_host=_cu([0, 10881]), num_seqs=1, H=16), -1, "fixed scratch"),
])
def test_forward_noalloc_rejects_before_any_hip_call(lib, kw, code, needle):
    # every argument, the workspace size included, is checked before the library looks up
    # its scratch array, so these fail the same way without a device
    assert _fwd_noalloc(lib, **kw) == code
    assert needle in lib.fp8attn_last_error().decode()
    assert lib.fp8attn_workspace_bytes(10881, 1, 16, 128) > (64 << 20)
    assert lib.fp8attn_workspace_bytes(10880, 1, 16, 128) == (64 << 20)
