"""ctypes loader for libfp8attn.so (built in-tree by fp8_dynamic_scaled_amd.build).

There is no fallback: if the library is missing or does not load, every entry point
raises. The signatures mirror include/fp8attn.h one to one.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libfp8attn.so")

FP8ATTN_OK = 0
FP8ATTN_EINVAL = -1
FP8ATTN_EUNSUPPORTED = -2
FP8ATTN_EHIP = -3
FP8ATTN_DYNAMIC = 0
FP8ATTN_STATIC = 1
FP8ATTN_SKIP = 1
FP8ATTN_OBSERVE = 2

_c_void_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
# host int32 tables (cu_seqlens_host) are passed by address as void pointers: the same ABI
# as const int32_t*, and an integer address avoids building a typed pointer per call
_host_i32 = ctypes.c_void_p
_f32p = ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes); every function declared in include/fp8attn.h
SIGNATURES = {
    "fp8attn_state_bytes": (ctypes.c_size_t, []),
    "fp8attn_state_reset": (ctypes.c_int, [_c_void_p, _c_void_p]),
    "fp8attn_observe_amax": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            ctypes.c_int64, _c_void_p]),
    "fp8attn_scales": (ctypes.c_int, [_c_void_p, ctypes.c_int, _f32p, ctypes.c_float,
                                      _c_void_p]),
    "fp8attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]),
    "fp8attn_quantize": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _host_i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _c_void_p, ctypes.c_size_t, _c_void_p]),
    "fp8attn_quantize_dynamic": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                _c_void_p, _host_i32, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, _c_void_p, ctypes.c_size_t,
                                                _c_void_p]),
    "fp8attn_forward": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _host_i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_uint, _c_void_p,
                                       ctypes.c_size_t, _c_void_p, _c_void_p]),
    "fp8attn_attend": (ctypes.c_int, [_c_void_p, _c_void_p, _host_i32, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_float, _c_void_p, ctypes.c_size_t,
                                      _c_void_p, _c_void_p]),
    "fp8attn_forward_noalloc": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                               _c_void_p, _host_i32, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_float, ctypes.c_uint,
                                               _c_void_p, _c_void_p]),
    "fp8attn_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libfp8attn.so once; raise with a clear message if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libfp8attn.so not found at {LIB_PATH}; build it with "
            "`python -m fp8_dynamic_scaled_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class Fp8AttnError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def check(fn_name, code):
    if code != FP8ATTN_OK:
        msg = load().fp8attn_last_error()
        raise Fp8AttnError(fn_name, code, msg.decode() if msg else "")
    return code
