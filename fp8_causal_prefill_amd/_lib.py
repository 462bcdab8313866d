"""ctypes declarations of the C ABI in include/zyfa.h (libzyfa.so, built in-tree)."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzyfa.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_LAUNCH = 3

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

_SIGNATURES = {
    "zyfa_abi_version": ([], _i),
    "zyfa_status_string": ([_i], ctypes.c_char_p),
    "zyfa_last_error": ([], ctypes.c_char_p),
    "zyfa_quantize_fp8": ([_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp], _i),
    "zyfa_attn_fwd_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "zyfa_attn_fwd_fp8_lean": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "zyfa_attn_fwd_bf16": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "zyfa_attn_fwd_fp8_range": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp] + [_i] * 10 + [_f, _i, _vp], _i),
    "zyfa_attn_fwd_bf16_range": ([_vp, _vp, _vp, _vp, _vp] + [_i] * 10 + [_f, _vp], _i),
    "zyfa_attn_merge": ([_vp, _vp, _i, _vp, _vp, ctypes.c_longlong, _i, _vp], _i),
    "zyfa_attn_fwd_fp8_varlen": ([_vp] * 6 + [_i, _vp, _vp, _vp] + [_i] * 7 + [_f, _i, _vp], _i),
    "zyfa_attn_fwd_bf16_varlen": ([_vp] * 6 + [_i] * 7 + [_f, _vp], _i),
    "zyfa_attn_fwd_fp8_paged": ([_vp] * 6 + [_i] + [_vp] * 5 + [_i] * 10 + [_f, _i, _vp], _i),
    "zyfa_attn_fwd_bf16_paged": ([_vp] * 8 + [_i] * 10 + [_f, _vp], _i),
    "zyfa_attn_decode_workspace_bytes": ([_i] * 5, ctypes.c_longlong),
    "zyfa_attn_decode_fp8_paged": ([_vp] * 6 + [_i] + [_vp] * 4 + [_i] * 9 + [_f, _i, _vp, ctypes.c_longlong, _i, _vp],
                                   _i),
    "zyfa_attn_decode_bf16_paged": ([_vp] * 7 + [_i] * 9 + [_f, _i, _vp, ctypes.c_longlong, _vp], _i),
    "zyfa_attn_decode_fp8_paged_noalloc": ([_vp] * 6 + [_i] + [_vp] * 4 + [_i] * 9 + [_f, _i, _i, _vp], _i),
}


class ZyfaError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load():
    """Load libzyfa.so (once). Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_causal_prefill_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(status: int, what: str):
    if status != OK:
        lib = load()
        msg = lib.zyfa_last_error().decode()
        name = lib.zyfa_status_string(status).decode()
        raise ZyfaError(status, f"{what}: {name}: {msg}")
