"""ctypes view of libawq.so (the C ABI declared in include/awq.h).

Loading fails loudly if the library has not been built: there is no fallback
implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libawq.so")

c_i32, c_i64, c_size, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/awq.h
SIGNATURES = {
    "awq_packed_bytes": (c_size, [c_i64, c_i64]),
    "awq_scales_bytes": (c_size, [c_i64, c_i64, c_i32]),
    "awq_zeros_bytes": (c_size, [c_i64, c_i64, c_i32]),
    "awq_quantize_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i32, c_i32]),
    "awq_channel_mean_abs": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "awq_pack": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "awq_quantize": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_i32,
                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "awq_gemm": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp]),
    "awq_unpack": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "awq_packed_bytes_bits": (c_size, [c_i64, c_i64, c_i32]),
    "awq_pack_bits": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "awq_quantize_bits": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_i32,
                                         c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "awq_quantize_shared": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_i32, c_i32,
                                           c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "awq_gemm_bits": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp]),
    "awq_gemm_kernel": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_i32, ctypes.c_char_p, c_size]),
    "awq_gemm_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i32]),
    "awq_gemm_ws": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_size, c_vp]),
    "awq_gemm_ws_kernel": (ctypes.c_int, [c_i64, c_i64, c_i64, c_i32, c_i32, ctypes.c_char_p, c_size]),
    "awq_unpack_bits": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "awq_ablation_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i32]),
    "awq_keep_fp16_ablation": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp,
                                              c_vp, c_vp, c_vp, c_size, c_vp]),
    "awq_scale_input": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "awq_gemm_scaled_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i32]),
    "awq_gemm_scaled": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32,
                                       c_vp, c_size, c_vp]),
    "awq_gemm_scaled_static": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32,
                                              c_vp]),
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_last_error": (ctypes.c_char_p, []),
    "awq_version": (ctypes.c_int, []),
}

_lib = None


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load() -> ctypes.CDLL:
    """Loads libawq.so once; raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != 0:
        lib = load()
        raise AwqError(status, f"{lib.awq_status_string(status).decode()}: {lib.awq_last_error().decode()}")
