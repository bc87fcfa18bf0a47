"""torch-facing binding of libfp8attn (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C-ABI; these functions
only check that tensors are what the C-ABI expects (device, dtype, contiguity), pass raw
pointers and the current HIP stream, and turn a non-OK status into an exception. torch is
used for device memory and streams.
"""
import ctypes
import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import FP8ATTN_DYNAMIC, FP8ATTN_OBSERVE, FP8ATTN_SKIP, FP8ATTN_STATIC, check

HEAD_DIM = 128
DEFAULT_MARGIN = 1.5
CUR_STRIPES = 16       # FP8ATTN_CUR_STRIPES
STATE_DTYPE = np.dtype([("ring", "<f4", (3, 16)), ("count", "<u4"),
                        ("scale", "<f4", (3,)), ("inv_scale", "<f4", (3,)),
                        ("amax", "<f4", (3,)), ("moved", "<u4"), ("reserved", "<u4", (5,)),
                        ("cur", "<u4", (CUR_STRIPES, 16))])


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _host_addr(a: np.ndarray) -> int:
    """Address of a host int32 table (the caller keeps the array alive for the call)."""
    return a.__array_interface__["data"][0]


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (device memory), got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_state(state):
    """A state must be a contiguous uint8 device tensor of at least fp8attn_state_bytes():
    the library only sees its address, so a shorter tensor would be written past its end."""
    _need_cuda("state", state, torch.uint8)
    if state.numel() < STATE_DTYPE.itemsize:
        raise ValueError(f"state must hold {STATE_DTYPE.itemsize} bytes, got {state.numel()}")


def _cu_host(cu_seqlens: torch.Tensor, cu_seqlens_host) -> np.ndarray:
    if cu_seqlens_host is None:
        # convenience path: one device -> host copy; pass the host copy to avoid it
        cu_seqlens_host = cu_seqlens.to("cpu")
    if isinstance(cu_seqlens_host, torch.Tensor):
        arr = cu_seqlens_host.to(torch.int32).contiguous().numpy()
    else:
        arr = np.asarray(cu_seqlens_host, dtype=np.int32)
    return np.ascontiguousarray(arr, dtype=np.int32)


def state_bytes() -> int:
    return int(_lib.load().fp8attn_state_bytes())


def workspace_bytes(total_tokens: int, num_seqs: int, num_heads: int,
                    head_dim: int = HEAD_DIM) -> int:
    return int(_lib.load().fp8attn_workspace_bytes(total_tokens, num_seqs, num_heads, head_dim))


def state_reset(state: torch.Tensor) -> None:
    _need_state(state)
    check("fp8attn_state_reset", _lib.load().fp8attn_state_reset(_ptr(state), _stream(state.device)))


def new_state(device=None) -> torch.Tensor:
    """A zeroed per-layer state (fp8attn_state_bytes() = 1280 bytes of device memory)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    st = torch.empty(state_bytes(), dtype=torch.uint8, device=device)
    state_reset(st)
    return st


def read_state(state: torch.Tensor) -> dict:
    """Host copy of a state's fields (synchronises with the state's stream)."""
    raw = state.detach().to("cpu").numpy().tobytes()
    rec = np.frombuffer(raw, dtype=STATE_DTYPE, count=1)[0]
    return {name: np.array(rec[name]) for name in STATE_DTYPE.names}


def observe_amax(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
    _need_state(state)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, torch.bfloat16)
    if not (q.numel() == k.numel() == v.numel()):
        raise ValueError("q, k and v must have the same number of elements")
    check("fp8attn_observe_amax",
          _lib.load().fp8attn_observe_amax(_ptr(state), _ptr(q), _ptr(k), _ptr(v), q.numel(),
                                           _stream(q.device)))


def scales(state: torch.Tensor, mode: str = "dynamic", static_amax: Optional[Sequence[float]] = None,
           margin: float = DEFAULT_MARGIN) -> None:
    _need_state(state)
    if mode == "dynamic":
        m, arr = FP8ATTN_DYNAMIC, None
    elif mode == "static":
        m = FP8ATTN_STATIC
        if static_amax is None or len(static_amax) != 3:
            raise ValueError("static mode needs static_amax = (q, k, v)")
        arr = (ctypes.c_float * 3)(*[float(x) for x in static_amax])
    else:
        raise ValueError(f"unknown scale mode {mode!r}")
    check("fp8attn_scales",
          _lib.load().fp8attn_scales(_ptr(state), m, arr, ctypes.c_float(margin),
                                     _stream(state.device)))


def _varlen_args(q, k, v, cu_seqlens, cu_seqlens_host):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, torch.bfloat16)
        if t.dim() != 3:
            raise ValueError(f"{name} must be [total_tokens, num_heads, head_dim]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    host = _cu_host(cu_seqlens, cu_seqlens_host)
    if host.shape[0] != cu_seqlens.numel():
        raise ValueError("cu_seqlens and cu_seqlens_host differ in length")
    T, H, D = q.shape
    if int(host[-1]) != T:
        raise ValueError(f"cu_seqlens[-1] = {int(host[-1])} but q has {T} tokens")
    return host, T, H, D


def quantize(state, q, k, v, cu_seqlens, cu_seqlens_host=None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Quantise into the FP8 workspace layout (Q8 | K8 | V8t); returns the workspace."""
    host, T, H, D = _varlen_args(q, k, v, cu_seqlens, cu_seqlens_host)
    _need_state(state)
    B = host.shape[0] - 1
    need = workspace_bytes(T, B, H, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need_cuda("workspace", workspace, torch.uint8)
    check("fp8attn_quantize",
          _lib.load().fp8attn_quantize(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                       _host_addr(host), B, H, D, _ptr(workspace),
                                       workspace.numel(), _stream(q.device)))
    return workspace


def quantize_dynamic(state, q, k, v, cu_seqlens, cu_seqlens_host=None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One dynamic forward's observe + ring + scales + quantise (fp8attn_quantize_dynamic):
    the same state and workspace bytes as observe_amax, scales("dynamic") and quantize,
    reading Q/K/V once when the window maximum does not move. Returns the workspace."""
    host, T, H, D = _varlen_args(q, k, v, cu_seqlens, cu_seqlens_host)
    B = host.shape[0] - 1
    need = workspace_bytes(T, B, H, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need_state(state)
    _need_cuda("workspace", workspace, torch.uint8)
    check("fp8attn_quantize_dynamic",
          _lib.load().fp8attn_quantize_dynamic(_ptr(state), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(cu_seqlens), _host_addr(host),
                                               B, H, D, _ptr(workspace), workspace.numel(),
                                               _stream(q.device)))
    return workspace


def split_workspace(workspace: torch.Tensor, total_tokens: int, num_seqs: int, num_heads: int,
                    head_dim: int = HEAD_DIM):
    """Views (q8 [T,H,D], k8 [T,H,D], v8t [H,D,Tp]) of a workspace (uint8)."""
    n = total_tokens * num_heads * head_dim
    Tp = (total_tokens + 127) // 128 * 128 + 128 * num_seqs
    q8 = workspace[:n].view(total_tokens, num_heads, head_dim)
    k8 = workspace[n:2 * n].view(total_tokens, num_heads, head_dim)
    v8t = workspace[2 * n:2 * n + num_heads * head_dim * Tp].view(num_heads, head_dim, Tp)
    return q8, k8, v8t


def pad_start(cu_i: int, i: int) -> int:
    """First padded key column of sequence i in V8t (see fp8attn.h)."""
    return (cu_i + 127) // 128 * 128 + 128 * i


def attend(state, workspace, cu_seqlens, cu_seqlens_host, num_heads: int,
           softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
           head_dim: int = HEAD_DIM) -> torch.Tensor:
    """FP8 attention on a workspace filled by quantize() (no quantisation step)."""
    _need_state(state)
    _need_cuda("workspace", workspace, torch.uint8)
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    host = _cu_host(cu_seqlens, cu_seqlens_host)
    T, B = int(host[-1]), host.shape[0] - 1
    if out is None:
        out = torch.empty((T, num_heads, head_dim), dtype=torch.bfloat16, device=workspace.device)
    _need_cuda("out", out, torch.bfloat16)
    if tuple(out.shape) != (T, num_heads, head_dim):
        raise ValueError("out must be [total_tokens, num_heads, head_dim]")
    check("fp8attn_attend",
          _lib.load().fp8attn_attend(_ptr(state), _ptr(cu_seqlens), _host_addr(host),
                                     B, num_heads, head_dim, ctypes.c_float(softmax_scale),
                                     _ptr(workspace), workspace.numel(), _ptr(out),
                                     _stream(workspace.device)))
    return out


def forward(state, q, k, v, cu_seqlens, cu_seqlens_host=None, softmax_scale: float = 0.0,
            skip: bool = False, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, observe: bool = False) -> torch.Tensor:
    """Varlen attention forward; FP8 path unless skip (then the BF16 kernel). With
    observe=True the FP8 path first does the dynamic observe + ring + scales update itself
    (FP8ATTN_OBSERVE)."""
    if skip and observe:
        raise ValueError("observe applies to the FP8 path only")
    host, T, H, D = _varlen_args(q, k, v, cu_seqlens, cu_seqlens_host)
    B = host.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    _need_cuda("out", out, torch.bfloat16)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    ws_n = 0
    if not skip:
        if state is None:
            raise ValueError("the FP8 path needs a state")
        _need_state(state)
        need = workspace_bytes(T, B, H, D)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _need_cuda("workspace", workspace, torch.uint8)
        ws_n = workspace.numel()
    flags = (FP8ATTN_SKIP if skip else 0) | (FP8ATTN_OBSERVE if observe else 0)
    check("fp8attn_forward",
          _lib.load().fp8attn_forward(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                      _host_addr(host), B, H, D,
                                      ctypes.c_float(softmax_scale), flags,
                                      _ptr(workspace if not skip else None), ws_n, _ptr(out),
                                      _stream(q.device)))
    return out


class AttentionLayer:
    """FP8 attention state of one attention layer.

    Dynamic (default): every FP8 forward observes the Q/K/V amax and updates the layer's
    16-slot ring before quantising -- by default in one pass over Q/K/V
    (fp8attn_quantize_dynamic, identical bytes); one_pass=False issues the separate
    observe, scales and quantise calls instead. Static: pass static_amax = calibrated
    (q, k, v) amax;
    the scale is amax * margin / 448 and nothing is observed. A forward with skip=True runs
    the BF16 kernel and leaves the state untouched.
    """

    def __init__(self, device=None, static_amax=None, margin: float = DEFAULT_MARGIN,
                 one_pass: bool = True):
        self.state = new_state(device)
        self.one_pass = bool(one_pass)
        self.static_amax = None if static_amax is None else [float(x) for x in static_amax]
        self.margin = float(margin)
        self._ws = None

    def workspace(self, T, B, H, device):
        need = max(workspace_bytes(T, B, H), 1)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def __call__(self, q, k, v, cu_seqlens, cu_seqlens_host=None, skip=False,
                 softmax_scale=0.0, out=None):
        if skip:
            return forward(None, q, k, v, cu_seqlens, cu_seqlens_host, softmax_scale, True,
                           None, out)
        host = _cu_host(cu_seqlens, cu_seqlens_host)
        ws = self.workspace(q.shape[0], host.shape[0] - 1, q.shape[1], q.device)
        if self.static_amax is None:
            if self.one_pass:
                return forward(self.state, q, k, v, cu_seqlens, host, softmax_scale, False, ws,
                               out, observe=True)
            observe_amax(self.state, q, k, v)
            scales(self.state, "dynamic")
        else:
            scales(self.state, "static", self.static_amax, self.margin)
        return forward(self.state, q, k, v, cu_seqlens, host, softmax_scale, False, ws, out)


def default_softmax_scale(head_dim: int = HEAD_DIM) -> float:
    """The binary32 value of 1/sqrt(head_dim) that the library uses for softmax_scale <= 0."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))
