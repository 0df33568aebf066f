"""The C++ oracle (oracle/awq_oracle.cpp, built into oracle/liboracle.so) behind numpy-facing
functions with the names and signatures of oracle/awq_oracle.py.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the bench's CPU-baseline
leg may import this module.  It marshals arrays (fp16 as raw 16-bit patterns) and calls the
library; every step of the method runs in the C++ code.  Loading fails loudly when the
library has not been built (`python -c 'import __graft_entry__ as g; g.build()'`).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCE = os.path.join(HERE, "awq_oracle.cpp")

# g++ flags: IEEE fp32/fp64 with no fused multiply-add (-ffp-contract=off, no fast-math);
# vectorised loops keep each sum's order; OpenMP only over independent rows.
CXXFLAGS = ["-O3", "-mavx2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c++17"]

_p, _i64, _i32, _f32, _f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
_SIGNATURES = {
    "oracle_f32_to_f16": (ctypes.c_uint16, [_f32]),
    "oracle_f16_to_f32": (_f32, [ctypes.c_uint16]),
    "oracle_channel_mean_abs": (None, [_p, _i64, _i64, _p]),
    "oracle_scales_for_alpha": (None, [_p, _i64, _f32, _p]),
    "oracle_scale_weights": (None, [_p, _p, _i64, _i64, _p]),
    "oracle_quantize_groups": (None, [_p, _i64, _i64, _i32, _i32, _p, _p, _p]),
    "oracle_dequantize": (None, [_p, _p, _p, _i64, _i64, _i32, _p]),
    "oracle_weight_error": (None, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _p]),
    "oracle_output_mse": (_f64, [_p, _i64, _i64, _p, _i64]),
    "oracle_gram": (None, [_p, _i64, _i64, _p]),
    "oracle_output_mse_gram": (_f64, [_p, _i64, _p, _i64, _i64]),
    "oracle_search": (None, [_p, _p, _i64, _i64, _i64, _i32, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "oracle_gemm": (None, [_p, _i64, _i64, _p, _p, _p, _i64, _i32, _p]),
    "oracle_scaled_input": (None, [_p, _i64, _i64, _p, _p]),
    "oracle_top_channels": (None, [_p, _i64, _i32, _p]),
    "oracle_keep_fp16_error": (None, [_p, _i64, _i64, _p, _i32, _i32, _i32, _p]),
    "oracle_keep_fp16_ablation": (None, [_p, _p, _i64, _i64, _i64, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
}

_lib = None


def build(out: str = LIB_PATH, source: str = SOURCE) -> str:
    """Compiles the C++ oracle with g++ into `out`."""
    import subprocess
    tmp = out + ".tmp"
    r = subprocess.run(["g++", *CXXFLAGS, source, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for {source}:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f16(a):
    """fp16 array as contiguous raw 16-bit patterns."""
    a = np.asarray(a)
    assert a.dtype == np.float16, f"expected float16, got {a.dtype}"
    return np.ascontiguousarray(a).view(np.uint16)


def alpha_grid(n: int = 20) -> np.ndarray:
    """alpha_i = i / n, i = 0..n-1, as float32 (a grid over [0, 1))."""
    return (np.arange(n, dtype=np.float32) / np.float32(n)).astype(np.float32)


def channel_mean_abs(X: np.ndarray) -> np.ndarray:
    Xb = _f16(X)
    M, K = Xb.shape
    a = np.empty(K, np.float64)
    load().oracle_channel_mean_abs(_ptr(Xb), M, K, _ptr(a))
    return a


def scales_for_alpha(a: np.ndarray, alpha) -> np.ndarray:
    a = _c(a, np.float64)
    s = np.empty(a.shape[0], np.float32)
    load().oracle_scales_for_alpha(_ptr(a), a.shape[0], float(np.float32(alpha)), _ptr(s))
    return s


def scale_weights(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    Wb = _f16(W)
    N, K = Wb.shape
    sv = _c(s, np.float32)
    V = np.empty((N, K), np.float32)
    load().oracle_scale_weights(_ptr(Wb), _ptr(sv), N, K, _ptr(V))
    return V


def quantize_groups(V: np.ndarray, group: int = 128, bits: int = 4):
    V = _c(V, np.float32)
    N, K = V.shape
    assert K % group == 0
    q = np.empty((N, K), np.uint8)
    z = np.empty((N, K // group), np.uint8)
    sc = np.empty((N, K // group), np.uint16)
    load().oracle_quantize_groups(_ptr(V), N, K, group, bits, _ptr(q), _ptr(z), _ptr(sc))
    return q, z, sc.view(np.float16)


def dequantize(q, z, sc16, group: int = 128) -> np.ndarray:
    q, z, sc = _c(q, np.uint8), _c(z, np.uint8), _f16(sc16)
    N, K = q.shape
    out = np.empty((N, K), np.float64)
    load().oracle_dequantize(_ptr(q), _ptr(z), _ptr(sc), N, K, group, _ptr(out))
    return out


def weight_error(W, q, z, sc16, s, group: int = 128) -> np.ndarray:
    Wb, q, z, sc = _f16(W), _c(q, np.uint8), _c(z, np.uint8), _f16(sc16)
    sv = None if s is None else _c(s, np.float32)
    N, K = q.shape
    E = np.empty((N, K), np.float64)
    load().oracle_weight_error(_ptr(Wb), _ptr(q), _ptr(z), _ptr(sc), _ptr(sv), N, K, group, _ptr(E))
    return E


def effective_weight(q, z, sc16, s, group: int = 128) -> np.ndarray:
    """w_hat / s along k in fp64: the weight error of an all-zero W."""
    return weight_error(np.zeros(np.shape(q), np.float16), q, z, sc16, s, group)


def output_mse(X: np.ndarray, E: np.ndarray) -> float:
    Xb, E = _f16(X), _c(E, np.float64)
    M, K = Xb.shape
    return float(load().oracle_output_mse(_ptr(Xb), M, K, _ptr(E), E.shape[0]))


def gram(X: np.ndarray) -> np.ndarray:
    Xb = _f16(X)
    M, K = Xb.shape
    G = np.empty((K, K), np.float64)
    load().oracle_gram(_ptr(Xb), M, K, _ptr(G))
    return G


def output_mse_gram(G: np.ndarray, E: np.ndarray, M: int) -> float:
    G, E = _c(G, np.float64), _c(E, np.float64)
    return float(load().oracle_output_mse_gram(_ptr(G), G.shape[0], _ptr(E), E.shape[0], int(M)))


def quantize_at(W, a, alpha, group: int = 128, bits: int = 4):
    s = scales_for_alpha(a, alpha)
    q, z, sc16 = quantize_groups(scale_weights(W, s), group, bits)
    return q, z, sc16, s


def search(W: np.ndarray, X: np.ndarray, group: int = 128, alphas=None, bits: int = 4,
           use_gram: bool | None = None) -> dict:
    Wb, Xb = _f16(W), _f16(X)
    N, K = Wb.shape
    M = Xb.shape[0]
    assert Xb.shape[1] == K
    al = _c(alpha_grid(20) if alphas is None else alphas, np.float32)
    n_alpha = al.shape[0]
    best = np.zeros(1, np.int32)
    losses = np.empty(n_alpha, np.float64)
    a = np.empty(K, np.float64)
    q = np.empty((N, K), np.uint8)
    z = np.empty((N, K // group), np.uint8)
    sc = np.empty((N, K // group), np.uint16)
    s = np.empty(K, np.float32)
    ug = -1 if use_gram is None else int(bool(use_gram))
    load().oracle_search(_ptr(Wb), _ptr(Xb), N, K, M, group, bits, _ptr(al), n_alpha, ug, _ptr(best), _ptr(losses),
                         _ptr(a), _ptr(q), _ptr(z), _ptr(sc), _ptr(s))
    b = int(best[0])
    return dict(alpha_index=b, alpha=float(al[b]), losses=losses, a=a, q=q, z=z, scales=sc.view(np.float16), s=s)


def top_channels(v: np.ndarray, n_keep: int) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(n_keep, np.int32)
    load().oracle_top_channels(_ptr(v), v.shape[0], n_keep, _ptr(out))
    return out


def keep_fp16_error(W: np.ndarray, keep, group: int = 128, bits: int = 4) -> np.ndarray:
    Wb = _f16(W)
    N, K = Wb.shape
    kp = _c(keep, np.int32)
    E = np.empty((N, K), np.float64)
    load().oracle_keep_fp16_error(_ptr(Wb), N, K, _ptr(kp), kp.shape[0], group, bits, _ptr(E))
    return E


def keep_fp16_ablation(W: np.ndarray, X: np.ndarray, n_keep: int, random_keep, group: int = 128,
                       bits: int = 4, use_gram: bool | None = None) -> dict:
    Wb, Xb = _f16(W), _f16(X)
    N, K = Wb.shape
    M = Xb.shape[0]
    rk = _c(random_keep, np.int32)
    assert rk.shape[0] == n_keep
    losses = np.empty(4, np.float64)
    ka, kw = np.empty(n_keep, np.int32), np.empty(n_keep, np.int32)
    a, b = np.empty(K, np.float64), np.empty(K, np.float64)
    ug = -1 if use_gram is None else int(bool(use_gram))
    load().oracle_keep_fp16_ablation(_ptr(Wb), _ptr(Xb), N, K, M, n_keep, _ptr(rk), group, bits, ug, _ptr(losses),
                                     _ptr(ka), _ptr(kw), _ptr(a), _ptr(b))
    return dict(losses=losses, keep_activation=ka, keep_weight=kw, a=a, b=b)


def scaled_input(x: np.ndarray, s) -> np.ndarray:
    xb = _f16(x)
    M, K = xb.shape
    sv = _c(s, np.float32)
    out = np.empty((M, K), np.uint16)
    load().oracle_scaled_input(_ptr(xb), M, K, _ptr(sv), _ptr(out))
    return out.view(np.float16)


def gemm(x: np.ndarray, q, z, sc16, group: int = 128) -> np.ndarray:
    xb, q, z, sc = _f16(x), _c(q, np.uint8), _c(z, np.uint8), _f16(sc16)
    M, K = xb.shape
    N = q.shape[0]
    y = np.empty((M, N), np.float64)
    load().oracle_gemm(_ptr(xb), M, K, _ptr(q), _ptr(z), _ptr(sc), N, group, _ptr(y))
    return y


def f32_to_f16_bits(f: float) -> int:
    """The oracle's own round-to-nearest-even fp32 -> fp16 conversion, as a bit pattern."""
    return int(load().oracle_f32_to_f16(float(np.float32(f))))
