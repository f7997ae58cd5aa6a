"""NVFP4 oracle: ctypes wrapper over ``nvfp4_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import it, and it imports nothing from them.

What it defines (Mix-Quant, Section 3.3 "NVFP4 Microscaling Quantization for
Prefilling", Eq. 2 and Eq. 3; see ``nvfp4_oracle.c`` for the FP32 readings):

* ``quantize(x_bf16)``      -> (codes, scales, alpha)   Eq. 3 then Eq. 2
* ``dequantize(...)``       -> float64 x_hat = alpha * sigma * q   (Eq. 2)
* ``gemm_exact(...)``       -> float64 Y = xhatA @ xhatW^T, exact int64 sum
* ``gemm_fp32(...)``        -> float32 Y from FP32 x_hat, products and k-ordered sums
* ``bf16_gemm(a, w)``       -> float64 Y of the BF16 decode path
* ``mx_quantize`` / ``mx_dequantize`` / ``mx_gemm``: MXFP4 (E2M1 + one E8M0
  power-of-two scale per 32), the coarser format Section 3.3 contrasts with
  NVFP4; rounding rule from the OCP MX v1.0 conversion (see nvfp4_oracle.c)

Function-level pins live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    I = ctypes.c_int
    sig = {
        "oracle_abi_version": (I, []),
        "oracle_default_threads": (I, []),
        "oracle_e2m1_value": (ctypes.c_double, [I]),
        "oracle_e4m3_value": (ctypes.c_double, [I]),
        "oracle_e2m1_encode": (I, [F]),
        "oracle_e4m3_encode": (I, [F]),
        "oracle_e2m1_encode_n": (None, [P, I64, P]),
        "oracle_e4m3_encode_n": (None, [P, I64, P]),
        "oracle_amax_bf16": (F, [P, I64, I64, I64]),
        "oracle_tensor_alpha": (F, [F]),
        "oracle_quantize": (I, [P, I64, I64, I64, I, P, P, P, I]),
        "oracle_quantize_f32": (I, [P, I64, I64, I64, I, P, P, P, I]),
        "oracle_dequantize": (None, [P, P, F, I64, I64, P]),
        "oracle_gemm_exact": (I, [P, P, F, P, P, F, I64, I64, I64, P, I]),
        "oracle_gemm_exact_pairs": (I, [P, P, F, P, P, F, I64, I64, I64, P, P, I64, P, I]),
        "oracle_gemm_fp32": (I, [P, P, F, P, P, F, I64, I64, I64, P, I]),
        "oracle_bf16_gemm": (None, [P, P, I64, I64, I64, P, I]),
        "oracle_bf16_gemm_pairs": (None, [P, P, I64, P, P, I64, P, I]),
        "oracle_e8m0_value": (ctypes.c_double, [I]),
        "oracle_mx_quantize": (I, [P, I64, I64, I64, P, P, I]),
        "oracle_mx_dequantize": (None, [P, P, I64, I64, P]),
        "oracle_mx_gemm": (I, [P, P, P, P, I64, I64, I64, P, I]),
        "oracle_mx_gemm_pairs": (I, [P, P, P, P, I64, P, P, I64, P, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def default_threads() -> int:
    return int(_load().oracle_default_threads())


# --------------------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def e2m1_table() -> np.ndarray:
    """Values of the 16 E2M1 codes (index = code)."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """Values of the 256 E4M3 codes (index = code; NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_encode(v) -> np.ndarray:
    v = _c(np.asarray(v, dtype=np.float32).ravel(), np.float32)
    out = np.empty(v.size, dtype=np.uint8)
    _load().oracle_e2m1_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode(s) -> np.ndarray:
    s = _c(np.asarray(s, dtype=np.float32).ravel(), np.float32)
    out = np.empty(s.size, dtype=np.uint8)
    _load().oracle_e4m3_encode_n(_ptr(s), s.size, _ptr(out))
    return out


# --------------------------------------------------------------------------- quantize
def tensor_alpha(amax: float) -> float:
    return float(_load().oracle_tensor_alpha(ctypes.c_float(amax)))


def amax_bf16(x_bits: np.ndarray) -> float:
    x = _c(x_bits, np.uint16)
    return float(_load().oracle_amax_bf16(_ptr(x), x.shape[0], x.shape[1], x.shape[1]))


def quantize(x_bits: np.ndarray, alpha: float | None = None, nthreads: int = 0):
    """Quantize a BF16 matrix given as uint16 bits [rows, cols].

    alpha=None computes the tensor scale from the data (dynamic); a float is
    used as a static tensor scale.  Returns (codes [rows, cols/2] uint8,
    scales [rows, cols/16] uint8, alpha float32).
    """
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)
    a = np.array([0.0 if alpha is None else alpha], dtype=np.float32)
    rc = _load().oracle_quantize(_ptr(x), rows, cols, cols, 0 if alpha is None else 1, _ptr(a),
                                 _ptr(codes), _ptr(scales), nthreads)
    if rc != 0:
        raise ValueError("oracle_quantize: cols must be a multiple of 16")
    return codes, scales, np.float32(a[0])


def quantize_f32(x: np.ndarray, alpha: float | None = None, nthreads: int = 0):
    """Quantize an FP32 matrix [rows, cols] (each value as it is, e.g. a GEMM
    output); alpha as in quantize().  Returns (codes, scales, alpha)."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)
    a = np.array([0.0 if alpha is None else alpha], dtype=np.float32)
    rc = _load().oracle_quantize_f32(_ptr(x), rows, cols, cols, 0 if alpha is None else 1, _ptr(a),
                                     _ptr(codes), _ptr(scales), nthreads)
    if rc != 0:
        raise ValueError("oracle_quantize_f32: cols must be a multiple of 16")
    return codes, scales, np.float32(a[0])


def dequantize(codes: np.ndarray, scales: np.ndarray, alpha: float) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, half * 2), dtype=np.float64)
    _load().oracle_dequantize(_ptr(codes), _ptr(scales), ctypes.c_float(alpha), rows, half * 2, _ptr(out))
    return out


# --------------------------------------------------------------------------- GEMM
def gemm_exact(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, nthreads: int = 0) -> np.ndarray:
    """Y[m, n] = sum_k xhatA[m, k] xhatW[n, k], exact, as float64 [M, N]."""
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    M, N, K = a_codes.shape[0], w_codes.shape[0], a_codes.shape[1] * 2
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_exact(_ptr(a_codes), _ptr(a_scales), ctypes.c_float(a_alpha), _ptr(w_codes),
                                   _ptr(w_scales), ctypes.c_float(w_alpha), M, N, K, _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_exact failed ({rc})")
    return out


def gemm_exact_pairs(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, mi, ni, nthreads: int = 0):
    """The exact GEMM at the given (mi[i], ni[i]) output positions."""
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    mi = _c(np.asarray(mi, dtype=np.int64), np.int64)
    ni = _c(np.asarray(ni, dtype=np.int64), np.int64)
    M, N, K = a_codes.shape[0], w_codes.shape[0], a_codes.shape[1] * 2
    out = np.empty(mi.size, dtype=np.float64)
    rc = _load().oracle_gemm_exact_pairs(_ptr(a_codes), _ptr(a_scales), ctypes.c_float(a_alpha), _ptr(w_codes),
                                         _ptr(w_scales), ctypes.c_float(w_alpha), M, N, K, _ptr(mi), _ptr(ni),
                                         mi.size, _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_exact_pairs failed ({rc})")
    return out


def gemm_fp32(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, nthreads: int = 0) -> np.ndarray:
    """Literal FP32-accumulated dequantized product, float32 [M, N]."""
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    M, N, K = a_codes.shape[0], w_codes.shape[0], a_codes.shape[1] * 2
    out = np.empty((M, N), dtype=np.float32)
    rc = _load().oracle_gemm_fp32(_ptr(a_codes), _ptr(a_scales), ctypes.c_float(a_alpha), _ptr(w_codes),
                                  _ptr(w_scales), ctypes.c_float(w_alpha), M, N, K, _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_fp32 failed ({rc})")
    return out


def bf16_gemm(a_bits: np.ndarray, w_bits: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Y = A W^T for BF16 A [M, K] and W [N, K] (uint16 bits), float64 sums."""
    a, w = _c(a_bits, np.uint16), _c(w_bits, np.uint16)
    M, K = a.shape
    N = w.shape[0]
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_bf16_gemm(_ptr(a), _ptr(w), M, N, K, _ptr(out), nthreads)
    return out


def bf16_gemm_pairs(a_bits, w_bits, mi, ni, nthreads: int = 0) -> np.ndarray:
    a, w = _c(a_bits, np.uint16), _c(w_bits, np.uint16)
    mi = _c(np.asarray(mi, dtype=np.int64), np.int64)
    ni = _c(np.asarray(ni, dtype=np.int64), np.int64)
    out = np.empty(mi.size, dtype=np.float64)
    _load().oracle_bf16_gemm_pairs(_ptr(a), _ptr(w), a.shape[1], _ptr(mi), _ptr(ni), mi.size, _ptr(out), nthreads)
    return out


# --------------------------------------------------------------------------- MXFP4
def e8m0_value(code: int) -> float:
    return float(_load().oracle_e8m0_value(int(code)))


def mx_quantize(x_bits: np.ndarray, nthreads: int = 0):
    """BF16 bits [rows, cols] -> (codes [rows, cols/2], E8M0 scales [rows, cols/32])."""
    x = _c(x_bits, np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    if _load().oracle_mx_quantize(_ptr(x), rows, cols, cols, _ptr(codes), _ptr(scales), nthreads) != 0:
        raise ValueError("oracle_mx_quantize: cols must be a multiple of 32")
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, half * 2), dtype=np.float64)
    _load().oracle_mx_dequantize(_ptr(codes), _ptr(scales), rows, half * 2, _ptr(out))
    return out


def mx_gemm(a_codes, a_scales, w_codes, w_scales, nthreads: int = 0) -> np.ndarray:
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    M, N, K = a_codes.shape[0], w_codes.shape[0], a_codes.shape[1] * 2
    out = np.empty((M, N), dtype=np.float64)
    if _load().oracle_mx_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K, _ptr(out),
                              nthreads) != 0:
        raise ValueError("oracle_mx_gemm: K must be a multiple of 32")
    return out


def mx_gemm_pairs(a_codes, a_scales, w_codes, w_scales, mi, ni, nthreads: int = 0) -> np.ndarray:
    a_codes, a_scales = _c(a_codes, np.uint8), _c(a_scales, np.uint8)
    w_codes, w_scales = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    mi = _c(np.asarray(mi, dtype=np.int64), np.int64)
    ni = _c(np.asarray(ni, dtype=np.int64), np.int64)
    out = np.empty(mi.size, dtype=np.float64)
    if _load().oracle_mx_gemm_pairs(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), a_codes.shape[1] * 2,
                                    _ptr(mi), _ptr(ni), mi.size, _ptr(out), nthreads) != 0:
        raise ValueError("oracle_mx_gemm_pairs: K must be a multiple of 32")
    return out
