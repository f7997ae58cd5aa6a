"""Python binding of the C ABI in ``include/nvfp4.h`` (ctypes).

Argument marshalling only: every step of the path runs in the gfx950 kernels
of ``libnvfp4.so``.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

NVFP4_OK, NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_EHIP, NVFP4_EWORKSPACE = 0, -1, -2, -3, -4
NVFP4_OUT_F32, NVFP4_OUT_BF16 = 0, 1
NVFP4_ALPHA_DYNAMIC, NVFP4_ALPHA_STATIC = 0, 1

_lib = None

_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = {
    "nvfp4_abi_version": (_I, []),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_quantize_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quantize": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _I, _P, _SZ, _P]),
    "nvfp4_gemm": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P]),
    "nvfp4_gemm_quant_out": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_quant_gemm_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quant_gemm": (_I, [_P, _I64, _P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "bf16_gemm": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _I64, _P]),
    "mxfp4_quantize": (_I, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "mxfp4_gemm": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P]),
}


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python nvfp4_prefill_gemm_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def last_error() -> str:
    return lib().nvfp4_last_error().decode()


def _check(fn: str, rc: int):
    if rc != NVFP4_OK:
        raise Nvfp4Error(fn, rc, last_error())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


_OUT = {torch.float32: NVFP4_OUT_F32, torch.bfloat16: NVFP4_OUT_BF16}


def quantize_workspace_size(rows: int, cols: int) -> int:
    return int(lib().nvfp4_quantize_workspace_size(rows, cols))


def nvfp4_quantize(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   alpha: torch.Tensor | None = None, static_alpha: bool = False,
                   workspace: torch.Tensor | None = None, stream=None):
    """BF16 [rows, cols] -> (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], alpha float32 [1]).

    static_alpha=True reads the tensor scale from ``alpha``; otherwise it is
    computed from the data and written there."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D row-major tensor")
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if alpha is None:
        if static_alpha:
            raise ValueError("static_alpha needs alpha")
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = 0
    if not static_alpha:
        ws_bytes = quantize_workspace_size(rows, cols)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=dev)
    rc = lib().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _ptr(alpha),
                              NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC, _ptr(workspace),
                              workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("nvfp4_quantize", rc)
    return codes, scales, alpha


def nvfp4_gemm(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, out: torch.Tensor | None = None,
               out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """Y [M, N] = dequant(A) @ dequant(W)^T from NVFP4 operands."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (w_codes, "w_codes"), (w_scales, "w_scales")):
        _dev(t, n, torch.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("A and W disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    rc = lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(w_codes), _ptr(w_scales),
                          _ptr(w_alpha), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0), _stream(stream))
    _check("nvfp4_gemm", rc)
    return out


def nvfp4_gemm_quant_out(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, y_alpha: torch.Tensor,
                         y_codes: torch.Tensor | None = None, y_scales: torch.Tensor | None = None, stream=None):
    """NVFP4 GEMM with an NVFP4 output (static output scale y_alpha, float32 [1]).
    Returns (y_codes uint8 [M, N/2], y_scales uint8 [M, N/16])."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (w_codes, "w_codes"), (w_scales, "w_scales")):
        _dev(t, n, torch.uint8)
    _dev(y_alpha, "y_alpha", torch.float32)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("A and W disagree on K")
    if y_codes is None:
        y_codes = torch.empty((M, N // 2), dtype=torch.uint8, device=a_codes.device)
    if y_scales is None:
        y_scales = torch.empty((M, N // 16), dtype=torch.uint8, device=a_codes.device)
    rc = lib().nvfp4_gemm_quant_out(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(w_codes), _ptr(w_scales),
                                    _ptr(w_alpha), M, N, K, _ptr(y_codes), _ptr(y_scales), _ptr(y_alpha),
                                    _stream(stream))
    _check("nvfp4_gemm_quant_out", rc)
    return y_codes, y_scales


def quant_gemm_workspace_size(M: int, K: int) -> int:
    return int(lib().nvfp4_quant_gemm_workspace_size(M, K))


def nvfp4_quant_gemm(x: torch.Tensor, w_codes, w_scales, w_alpha, a_alpha: torch.Tensor | None = None,
                     static_alpha: bool = False, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                     workspace: torch.Tensor | None = None, stream=None):
    """Fused prefill linear: BF16 x quantized to NVFP4 inside the GEMM.  Returns (out, a_alpha)."""
    _dev(x, "x", torch.bfloat16)
    M, K = x.shape
    N = w_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if a_alpha is None:
        if static_alpha:
            raise ValueError("static_alpha needs a_alpha")
        a_alpha = torch.empty(1, dtype=torch.float32, device=x.device)
    ws_bytes = 0
    if not static_alpha:
        ws_bytes = quant_gemm_workspace_size(M, K)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=x.device)
    rc = lib().nvfp4_quant_gemm(_ptr(x), x.stride(0), _ptr(a_alpha),
                                NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC, _ptr(w_codes),
                                _ptr(w_scales), _ptr(w_alpha), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0),
                                _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("nvfp4_quant_gemm", rc)
    return out, a_alpha


def bf16_gemm(a: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
              stream=None) -> torch.Tensor:
    """Y [M, N] = A [M, K] @ W [N, K]^T in BF16 with FP32 accumulation."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    if not (a.is_contiguous() and w.is_contiguous()):
        raise ValueError("a and w must be contiguous")
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    rc = lib().bf16_gemm(_ptr(a), _ptr(w), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0), _stream(stream))
    _check("bf16_gemm", rc)
    return out


def mxfp4_quantize(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   stream=None):
    """BF16 [rows, cols] -> MXFP4 (codes uint8 [rows, cols/2], E8M0 scales uint8 [rows, cols/32])."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D row-major tensor")
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    rc = lib().mxfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _stream(stream))
    _check("mxfp4_quantize", rc)
    return codes, scales


def mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
               stream=None) -> torch.Tensor:
    """Y [M, N] = dequant(A) @ dequant(W)^T from MXFP4 operands."""
    for t, n in ((a_codes, "a_codes"), (a_scales, "a_scales"), (w_codes, "w_codes"), (w_scales, "w_scales")):
        _dev(t, n, torch.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("A and W disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    rc = lib().mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K, _ptr(out),
                          _OUT[out.dtype], out.stride(0), _stream(stream))
    _check("mxfp4_gemm", rc)
    return out
