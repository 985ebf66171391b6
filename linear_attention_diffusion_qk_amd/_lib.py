"""ctypes loader for libsanala.so: the C-ABI declared in include/sanala.h.

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsanala.so")

SANA_OK = 0
SANA_ERR_INVALID_ARG = 1
SANA_ERR_UNSUPPORTED = 2
SANA_ERR_MISALIGNED = 3
SANA_ERR_HIP = 4
SANA_ERR_SCRATCH_LIMIT = 5
SANA_F32 = 0
SANA_BF16 = 1
SANA_F16 = 2

# Every symbol include/sanala.h declares.
EXPORTS = ("sana_linear_attn_fwd", "sana_linear_attn_fwd_noalloc", "sana_qkv_linear_attn_fwd", "sana_qkv_w8a8_linear_attn_fwd",
           "sana_quantize_rows_i8", "sana_pack_weight_i8", "sana_mix_ffn_fwd", "sana_cross_attn_fwd", "sana_release_scratch",
           "sana_status_string", "sana_timing_enable", "sana_timing_last")

_lock = threading.Lock()
_lib = None


class SanaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: libsanala status {status} ({status_string(status)})")


def load_library() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_diffusion_qk_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.sana_linear_attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, vp, vp, ci]
        lib.sana_linear_attn_fwd.restype = ci
        lib.sana_linear_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, vp, vp, ci]
        lib.sana_linear_attn_fwd_noalloc.restype = ci
        lib.sana_qkv_linear_attn_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, vp, vp]
        lib.sana_qkv_linear_attn_fwd.restype = ci
        lib.sana_qkv_w8a8_linear_attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, vp, vp]
        lib.sana_qkv_w8a8_linear_attn_fwd.restype = ci
        lib.sana_quantize_rows_i8.argtypes = [vp, ctypes.c_int64, ci, vp, vp, vp]
        lib.sana_quantize_rows_i8.restype = ci
        lib.sana_pack_weight_i8.argtypes = [vp, ctypes.c_int64, ci, vp, vp]
        lib.sana_pack_weight_i8.restype = ci
        lib.sana_mix_ffn_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp]
        lib.sana_mix_ffn_fwd.restype = ci
        lib.sana_cross_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp, vp, ci]
        lib.sana_cross_attn_fwd.restype = ci
        lib.sana_release_scratch.argtypes = [vp]
        lib.sana_release_scratch.restype = ci
        lib.sana_status_string.argtypes = [ci]
        lib.sana_status_string.restype = ctypes.c_char_p
        lib.sana_timing_enable.argtypes = [ci]
        lib.sana_timing_enable.restype = ci
        lib.sana_timing_last.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), ci]
        lib.sana_timing_last.restype = ci
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().sana_status_string(int(status)).decode()


def library_path() -> str:
    return LIB_PATH
