"""Python binding of the C ABI in ``include/nvfp4.h`` (ctypes).

Argument marshalling only: every step of the path runs in the gfx950 kernels
of ``libnvfp4.so``.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

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
    "nvfp4_quantize_noalloc": (_I, [_P, _I64, _I64, _I64, _P, _P, _P, _I, _P]),
    "nvfp4_gemm_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_gemm": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "nvfp4_gemm_quant_out": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_gemm_quant_out_dynamic_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_gemm_quant_out_dynamic": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_quant_gemm_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_quant_gemm": (_I, [_P, _I64, _P, _I, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "nvfp4_decode_pack_size": (_SZ, [_I64, _I64]),
    "nvfp4_decode_pack": (_I, [_P, _P, _I64, _I64, _P, _P]),
    "nvfp4_gemm_packed": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "nvfp4_quant_gemm_packed": (_I, [_P, _I64, _P, _I, _P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "bf16_gemm_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "bf16_decode_pack_size": (_SZ, [_I64, _I64]),
    "bf16_decode_pack": (_I, [_P, _I64, _I64, _P, _P]),
    "bf16_gemm_packed": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "bf16_gemm": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
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
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# Argument checks run before any C call: the C ABI sees only pointers and
# sizes, so a tensor whose shape, dtype, layout or device disagrees with the
# sizes passed would make the kernels read or write outside it.  Shapes,
# dtypes and layouts are checked first, devices last.

def _tensor(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _mat(t, name: str, dtype, rows: int | None = None, cols: int | None = None, contiguous: bool = True):
    """2-D tensor of ``dtype`` with the given shape; row-major (contiguous, or
    rows of unit element stride when ``contiguous`` is False)."""
    _tensor(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name} must have {rows} rows, got shape {tuple(t.shape)}")
    if cols is not None and t.shape[1] != cols:
        raise ValueError(f"{name} must have {cols} columns, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and t.shape[0] > 1 and t.shape[1] > 0 and (t.stride(1) != 1 or t.stride(0) < t.shape[1]):
        raise ValueError(f"{name} must be row-major with unit column stride")
    return t


def _alpha(t, name: str):
    _tensor(t, name)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.numel() < 1:
        raise ValueError(f"{name} must hold at least one element")
    return t


def _out(t, name: str, rows: int, cols: int):
    """GEMM output [rows, cols], FP32 or BF16, unit column stride (row stride >= cols)."""
    _tensor(t, name)
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    if rows > 0 and cols > 0 and (t.stride(1) != 1 or (rows > 1 and t.stride(0) < cols)):
        raise ValueError(f"{name} must be row-major with unit column stride")
    return t


def _k_of_codes(codes: torch.Tensor, name: str, multiple: int = 16) -> int:
    k = codes.shape[1] * 2
    if k % multiple:
        raise ValueError(f"{name}: K = {k} must be a multiple of {multiple}")
    return k


def _same_device(*named):
    """Every tensor on the GPU, and all on one device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


_OUT = {torch.float32: NVFP4_OUT_F32, torch.bfloat16: NVFP4_OUT_BF16}


def quantize_workspace_size(rows: int, cols: int) -> int:
    return int(lib().nvfp4_quantize_workspace_size(rows, cols))


def nvfp4_quantize(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   alpha: torch.Tensor | None = None, static_alpha: bool = False,
                   workspace: torch.Tensor | None = None, stream=None):
    """BF16 [rows, cols] -> (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], alpha float32 [1]).

    static_alpha=True reads the tensor scale from ``alpha``; otherwise it is
    computed from the data and written there."""
    _mat(x, "x", torch.bfloat16, contiguous=False)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError(f"x: cols = {cols} must be a multiple of 16")
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    if alpha is None:
        if static_alpha:
            raise ValueError("static_alpha needs alpha")
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    _mat(codes, "codes", torch.uint8, rows, cols // 2)
    _mat(scales, "scales", torch.uint8, rows, cols // 16)
    _alpha(alpha, "alpha")
    if workspace is not None:
        _tensor(workspace, "workspace")
    _same_device(("x", x), ("codes", codes), ("scales", scales), ("alpha", alpha), ("workspace", workspace))
    if not static_alpha and workspace is None:
        workspace = torch.empty(max(quantize_workspace_size(rows, cols), 4), dtype=torch.uint8, device=dev)
    rc = lib().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _ptr(alpha),
                              NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC, _ptr(workspace),
                              _nbytes(workspace), _stream(stream))
    _check("nvfp4_quantize", rc)
    return codes, scales, alpha


def nvfp4_quantize_noalloc(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, alpha: torch.Tensor,
                           static_alpha: bool = False, stream=None):
    """nvfp4_quantize into caller-provided outputs without a workspace: the
    dynamic tensor scale's partial maxima use the library's per-GPU scratch
    array (calls that overlap on one GPU race)."""
    _mat(x, "x", torch.bfloat16, contiguous=False)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError(f"x: cols = {cols} must be a multiple of 16")
    _mat(codes, "codes", torch.uint8, rows, cols // 2)
    _mat(scales, "scales", torch.uint8, rows, cols // 16)
    _alpha(alpha, "alpha")
    _same_device(("x", x), ("codes", codes), ("scales", scales), ("alpha", alpha))
    rc = lib().nvfp4_quantize_noalloc(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _ptr(alpha),
                                      NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC,
                                      _stream(stream))
    _check("nvfp4_quantize_noalloc", rc)
    return codes, scales, alpha


def _nvfp4_operands(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha):
    """Check both NVFP4 operands; returns (M, N, K)."""
    _mat(a_codes, "a_codes", torch.uint8)
    _mat(w_codes, "w_codes", torch.uint8)
    K = _k_of_codes(a_codes, "a_codes")
    if w_codes.shape[1] * 2 != K:
        raise ValueError(f"A and W disagree on K ({K} vs {w_codes.shape[1] * 2})")
    M, N = a_codes.shape[0], w_codes.shape[0]
    _mat(a_scales, "a_scales", torch.uint8, M, K // 16)
    _mat(w_scales, "w_scales", torch.uint8, N, K // 16)
    _alpha(a_alpha, "a_alpha")
    _alpha(w_alpha, "w_alpha")
    return M, N, K


def gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_gemm_workspace_size(M, N, K))


def bf16_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().bf16_gemm_workspace_size(M, N, K))


def _workspace(workspace, nbytes: int, dev):
    """The caller's workspace, or a fresh one of nbytes (None when 0).  Pass
    workspace=False to run without one."""
    if workspace is False:
        return None
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else None
    return _tensor(workspace, "workspace")


def nvfp4_gemm(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, out: torch.Tensor | None = None,
               out_dtype=torch.bfloat16, workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] = dequant(A) @ dequant(W)^T from NVFP4 operands.  workspace:
    device scratch (default: gemm_workspace_size bytes; False: none)."""
    M, N, K = _nvfp4_operands(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _out(out, "out", M, N)
    _same_device(("a_codes", a_codes), ("a_scales", a_scales), ("a_alpha", a_alpha), ("w_codes", w_codes),
                 ("w_scales", w_scales), ("w_alpha", w_alpha), ("out", out),
                 ("workspace", workspace if isinstance(workspace, torch.Tensor) else None))
    workspace = _workspace(workspace, gemm_workspace_size(M, N, K) if workspace is None else 0, a_codes.device)
    rc = lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(w_codes), _ptr(w_scales),
                          _ptr(w_alpha), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0), _ptr(workspace),
                          _nbytes(workspace), _stream(stream))
    _check("nvfp4_gemm", rc)
    return out


def nvfp4_gemm_quant_out(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, y_alpha: torch.Tensor,
                         y_codes: torch.Tensor | None = None, y_scales: torch.Tensor | None = None, stream=None):
    """NVFP4 GEMM with an NVFP4 output (static output scale y_alpha, float32 [1]).
    Returns (y_codes uint8 [M, N/2], y_scales uint8 [M, N/16])."""
    M, N, K = _nvfp4_operands(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha)
    if N % 16:
        raise ValueError(f"N = {N} must be a multiple of 16 for an NVFP4 output")
    _alpha(y_alpha, "y_alpha")
    if y_codes is None:
        y_codes = torch.empty((M, N // 2), dtype=torch.uint8, device=a_codes.device)
    if y_scales is None:
        y_scales = torch.empty((M, N // 16), dtype=torch.uint8, device=a_codes.device)
    _mat(y_codes, "y_codes", torch.uint8, M, N // 2)
    _mat(y_scales, "y_scales", torch.uint8, M, N // 16)
    _same_device(("a_codes", a_codes), ("a_scales", a_scales), ("a_alpha", a_alpha), ("w_codes", w_codes),
                 ("w_scales", w_scales), ("w_alpha", w_alpha), ("y_alpha", y_alpha), ("y_codes", y_codes),
                 ("y_scales", y_scales))
    rc = lib().nvfp4_gemm_quant_out(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(w_codes), _ptr(w_scales),
                                    _ptr(w_alpha), M, N, K, _ptr(y_codes), _ptr(y_scales), _ptr(y_alpha),
                                    _stream(stream))
    _check("nvfp4_gemm_quant_out", rc)
    return y_codes, y_scales


def gemm_quant_out_dynamic_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_gemm_quant_out_dynamic_workspace_size(M, N, K))


def nvfp4_gemm_quant_out_dynamic(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha,
                                 y_codes: torch.Tensor | None = None, y_scales: torch.Tensor | None = None,
                                 y_alpha: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                 stream=None):
    """NVFP4 GEMM with an NVFP4 output whose tensor scale comes from the
    output's own amax.  Returns (y_codes uint8 [M, N/2], y_scales uint8
    [M, N/16], y_alpha float32 [1])."""
    M, N, K = _nvfp4_operands(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha)
    if N % 16:
        raise ValueError(f"N = {N} must be a multiple of 16 for an NVFP4 output")
    dev = a_codes.device
    if y_codes is None:
        y_codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if y_scales is None:
        y_scales = torch.empty((M, N // 16), dtype=torch.uint8, device=dev)
    if y_alpha is None:
        y_alpha = torch.empty(1, dtype=torch.float32, device=dev)
    _mat(y_codes, "y_codes", torch.uint8, M, N // 2)
    _mat(y_scales, "y_scales", torch.uint8, M, N // 16)
    _alpha(y_alpha, "y_alpha")
    if workspace is None:
        workspace = torch.empty(max(gemm_quant_out_dynamic_workspace_size(M, N, K), 256), dtype=torch.uint8,
                                device=dev)
    _tensor(workspace, "workspace")
    _same_device(("a_codes", a_codes), ("a_scales", a_scales), ("a_alpha", a_alpha), ("w_codes", w_codes),
                 ("w_scales", w_scales), ("w_alpha", w_alpha), ("y_alpha", y_alpha), ("y_codes", y_codes),
                 ("y_scales", y_scales), ("workspace", workspace))
    rc = lib().nvfp4_gemm_quant_out_dynamic(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(w_codes),
                                            _ptr(w_scales), _ptr(w_alpha), M, N, K, _ptr(y_codes), _ptr(y_scales),
                                            _ptr(y_alpha), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("nvfp4_gemm_quant_out_dynamic", rc)
    return y_codes, y_scales, y_alpha


def quant_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_quant_gemm_workspace_size(M, N, K))


def nvfp4_quant_gemm(x: torch.Tensor, w_codes, w_scales, w_alpha, a_alpha: torch.Tensor | None = None,
                     static_alpha: bool = False, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                     workspace: torch.Tensor | None = None, stream=None):
    """Fused prefill linear: BF16 x quantized to NVFP4 inside the GEMM.  Returns (out, a_alpha)."""
    _mat(x, "x", torch.bfloat16, contiguous=False)
    M, K = x.shape
    if K % 16:
        raise ValueError(f"x: K = {K} must be a multiple of 16")
    _mat(w_codes, "w_codes", torch.uint8, cols=K // 2)
    N = w_codes.shape[0]
    _mat(w_scales, "w_scales", torch.uint8, N, K // 16)
    _alpha(w_alpha, "w_alpha")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _out(out, "out", M, N)
    if a_alpha is None:
        if static_alpha:
            raise ValueError("static_alpha needs a_alpha")
        a_alpha = torch.empty(1, dtype=torch.float32, device=x.device)
    _alpha(a_alpha, "a_alpha")
    if workspace is not None:
        _tensor(workspace, "workspace")
    _same_device(("x", x), ("w_codes", w_codes), ("w_scales", w_scales), ("w_alpha", w_alpha), ("out", out),
                 ("a_alpha", a_alpha), ("workspace", workspace))
    if workspace is None:
        workspace = torch.empty(max(quant_gemm_workspace_size(M, N, K), 16), dtype=torch.uint8, device=x.device)
    rc = lib().nvfp4_quant_gemm(_ptr(x), x.stride(0), _ptr(a_alpha),
                                NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC, _ptr(w_codes),
                                _ptr(w_scales), _ptr(w_alpha), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0),
                                _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("nvfp4_quant_gemm", rc)
    return out, a_alpha


class DecodePackedWeight(NamedTuple):
    """An NVFP4 weight [N, K] in the decode-packed layout (include/nvfp4.h):
    ``packed`` uint8 [decode_pack_size(N, K)], ``alpha`` float32 [1]."""
    packed: torch.Tensor
    alpha: torch.Tensor
    n: int
    k: int


def decode_pack_size(N: int, K: int) -> int:
    return int(lib().nvfp4_decode_pack_size(N, K))


def _packed_weight(wp, K: int | None = None):
    if not isinstance(wp, DecodePackedWeight):
        raise TypeError(f"the weight must be a DecodePackedWeight, got {type(wp).__name__}")
    if K is not None and wp.k != K:
        raise ValueError(f"activations and the packed weight disagree on K ({K} vs {wp.k})")
    if wp.k % 128:
        raise ValueError(f"packed weight: K = {wp.k} must be a multiple of 128")
    _tensor(wp.packed, "packed")
    if wp.packed.dtype != torch.uint8 or wp.packed.dim() != 1 or not wp.packed.is_contiguous():
        raise ValueError("packed must be a contiguous 1-D uint8 tensor")
    if wp.packed.numel() != decode_pack_size(wp.n, wp.k):
        raise ValueError(f"packed holds {wp.packed.numel()} bytes, the layout of [{wp.n}, {wp.k}] takes "
                         f"{decode_pack_size(wp.n, wp.k)}")
    _alpha(wp.alpha, "w_alpha")
    return wp


def nvfp4_decode_pack(w_codes, w_scales, w_alpha, packed: torch.Tensor | None = None,
                      stream=None) -> DecodePackedWeight:
    """Row-major NVFP4 weight (codes [N, K/2], scales [N, K/16], alpha [1]) ->
    the decode-packed layout the *_packed GEMMs stream (K % 128 == 0)."""
    _mat(w_codes, "w_codes", torch.uint8)
    K = _k_of_codes(w_codes, "w_codes", 128)
    N = w_codes.shape[0]
    _mat(w_scales, "w_scales", torch.uint8, N, K // 16)
    _alpha(w_alpha, "w_alpha")
    if packed is None:
        packed = torch.empty(decode_pack_size(N, K), dtype=torch.uint8, device=w_codes.device)
    wp = _packed_weight(DecodePackedWeight(packed, w_alpha, N, K))
    _same_device(("w_codes", w_codes), ("w_scales", w_scales), ("w_alpha", w_alpha), ("packed", packed))
    rc = lib().nvfp4_decode_pack(_ptr(w_codes), _ptr(w_scales), N, K, _ptr(packed), _stream(stream))
    _check("nvfp4_decode_pack", rc)
    return wp


def nvfp4_gemm_packed(a_codes, a_scales, a_alpha, wp: DecodePackedWeight, out: torch.Tensor | None = None,
                      out_dtype=torch.bfloat16, workspace=None, stream=None) -> torch.Tensor:
    """nvfp4_gemm on a decode-packed weight (M <= 64)."""
    _mat(a_codes, "a_codes", torch.uint8)
    K = _k_of_codes(a_codes, "a_codes")
    M = a_codes.shape[0]
    _mat(a_scales, "a_scales", torch.uint8, M, K // 16)
    _alpha(a_alpha, "a_alpha")
    _packed_weight(wp, K)
    N = wp.n
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _out(out, "out", M, N)
    _same_device(("a_codes", a_codes), ("a_scales", a_scales), ("a_alpha", a_alpha), ("packed", wp.packed),
                 ("w_alpha", wp.alpha), ("out", out),
                 ("workspace", workspace if isinstance(workspace, torch.Tensor) else None))
    workspace = _workspace(workspace, gemm_workspace_size(M, N, K) if workspace is None else 0, a_codes.device)
    rc = lib().nvfp4_gemm_packed(_ptr(a_codes), _ptr(a_scales), _ptr(a_alpha), _ptr(wp.packed), _ptr(wp.alpha),
                                 M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream))
    _check("nvfp4_gemm_packed", rc)
    return out


def nvfp4_quant_gemm_packed(x: torch.Tensor, wp: DecodePackedWeight, a_alpha: torch.Tensor | None = None,
                            static_alpha: bool = False, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                            workspace: torch.Tensor | None = None, stream=None):
    """nvfp4_quant_gemm on a decode-packed weight (M <= 64).  Returns (out, a_alpha)."""
    _mat(x, "x", torch.bfloat16, contiguous=False)
    M, K = x.shape
    _packed_weight(wp, K)
    N = wp.n
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _out(out, "out", M, N)
    if a_alpha is None:
        if static_alpha:
            raise ValueError("static_alpha needs a_alpha")
        a_alpha = torch.empty(1, dtype=torch.float32, device=x.device)
    _alpha(a_alpha, "a_alpha")
    if workspace is not None:
        _tensor(workspace, "workspace")
    _same_device(("x", x), ("packed", wp.packed), ("w_alpha", wp.alpha), ("out", out), ("a_alpha", a_alpha),
                 ("workspace", workspace))
    if workspace is None:
        workspace = torch.empty(max(quant_gemm_workspace_size(M, N, K), 16), dtype=torch.uint8, device=x.device)
    rc = lib().nvfp4_quant_gemm_packed(_ptr(x), x.stride(0), _ptr(a_alpha),
                                       NVFP4_ALPHA_STATIC if static_alpha else NVFP4_ALPHA_DYNAMIC,
                                       _ptr(wp.packed), _ptr(wp.alpha), M, N, K, _ptr(out), _OUT[out.dtype],
                                       out.stride(0), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("nvfp4_quant_gemm_packed", rc)
    return out, a_alpha


def bf16_gemm(a: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
              workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] = A [M, K] @ W [N, K]^T in BF16 with FP32 accumulation.
    workspace: device scratch (default: bf16_gemm_workspace_size bytes; False: none)."""
    _mat(a, "a", torch.bfloat16)
    M, K = a.shape
    _mat(w, "w", torch.bfloat16, cols=K)
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _out(out, "out", M, N)
    _same_device(("a", a), ("w", w), ("out", out),
                 ("workspace", workspace if isinstance(workspace, torch.Tensor) else None))
    workspace = _workspace(workspace, bf16_gemm_workspace_size(M, N, K) if workspace is None else 0, a.device)
    rc = lib().bf16_gemm(_ptr(a), _ptr(w), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0), _ptr(workspace),
                         _nbytes(workspace), _stream(stream))
    _check("bf16_gemm", rc)
    return out


def mxfp4_quantize(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   stream=None):
    """BF16 [rows, cols] -> MXFP4 (codes uint8 [rows, cols/2], E8M0 scales uint8 [rows, cols/32])."""
    _mat(x, "x", torch.bfloat16, contiguous=False)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError(f"x: cols = {cols} must be a multiple of 32")
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _mat(codes, "codes", torch.uint8, rows, cols // 2)
    _mat(scales, "scales", torch.uint8, rows, cols // 32)
    _same_device(("x", x), ("codes", codes), ("scales", scales))
    rc = lib().mxfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _stream(stream))
    _check("mxfp4_quantize", rc)
    return codes, scales


def mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, out: torch.Tensor | None = None, out_dtype=torch.bfloat16,
               stream=None) -> torch.Tensor:
    """Y [M, N] = dequant(A) @ dequant(W)^T from MXFP4 operands."""
    _mat(a_codes, "a_codes", torch.uint8)
    _mat(w_codes, "w_codes", torch.uint8)
    K = _k_of_codes(a_codes, "a_codes", 32)
    if w_codes.shape[1] * 2 != K:
        raise ValueError(f"A and W disagree on K ({K} vs {w_codes.shape[1] * 2})")
    M, N = a_codes.shape[0], w_codes.shape[0]
    _mat(a_scales, "a_scales", torch.uint8, M, K // 32)
    _mat(w_scales, "w_scales", torch.uint8, N, K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    _out(out, "out", M, N)
    _same_device(("a_codes", a_codes), ("a_scales", a_scales), ("w_codes", w_codes), ("w_scales", w_scales),
                 ("out", out))
    rc = lib().mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K, _ptr(out),
                          _OUT[out.dtype], out.stride(0), _stream(stream))
    _check("mxfp4_gemm", rc)
    return out


class Bf16PackedWeight(NamedTuple):
    """A BF16 weight [N, K] in the decode-packed layout (include/nvfp4.h):
    ``packed`` uint8 [bf16_decode_pack_size(N, K)]."""
    packed: torch.Tensor
    n: int
    k: int


def bf16_decode_pack_size(N: int, K: int) -> int:
    return int(lib().bf16_decode_pack_size(N, K))


def bf16_decode_pack(w: torch.Tensor, packed: torch.Tensor | None = None, stream=None) -> Bf16PackedWeight:
    """Row-major BF16 weight [N, K] -> the decode-packed layout bf16_gemm_packed
    streams (K % 32 == 0)."""
    _mat(w, "w", torch.bfloat16)
    N, K = w.shape
    if K % 32:
        raise ValueError(f"w: K = {K} must be a multiple of 32")
    if packed is None:
        packed = torch.empty(bf16_decode_pack_size(N, K), dtype=torch.uint8, device=w.device)
    wp = _bf16_packed(Bf16PackedWeight(packed, N, K))
    _same_device(("w", w), ("packed", packed))
    rc = lib().bf16_decode_pack(_ptr(w), N, K, _ptr(packed), _stream(stream))
    _check("bf16_decode_pack", rc)
    return wp


def _bf16_packed(wp, K: int | None = None):
    if not isinstance(wp, Bf16PackedWeight):
        raise TypeError(f"the weight must be a Bf16PackedWeight, got {type(wp).__name__}")
    if K is not None and wp.k != K:
        raise ValueError(f"activations and the packed weight disagree on K ({K} vs {wp.k})")
    if wp.k % 32:
        raise ValueError(f"packed weight: K = {wp.k} must be a multiple of 32")
    _tensor(wp.packed, "packed")
    if wp.packed.dtype != torch.uint8 or wp.packed.dim() != 1 or not wp.packed.is_contiguous():
        raise ValueError("packed must be a contiguous 1-D uint8 tensor")
    if wp.packed.numel() != bf16_decode_pack_size(wp.n, wp.k):
        raise ValueError(f"packed holds {wp.packed.numel()} bytes, the layout of [{wp.n}, {wp.k}] takes "
                         f"{bf16_decode_pack_size(wp.n, wp.k)}")
    return wp


def bf16_gemm_packed(a: torch.Tensor, wp: Bf16PackedWeight, out: torch.Tensor | None = None,
                     out_dtype=torch.bfloat16, workspace=None, stream=None) -> torch.Tensor:
    """bf16_gemm on a decode-packed weight (M <= 64)."""
    _mat(a, "a", torch.bfloat16)
    M, K = a.shape
    _bf16_packed(wp, K)
    N = wp.n
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _out(out, "out", M, N)
    _same_device(("a", a), ("packed", wp.packed), ("out", out),
                 ("workspace", workspace if isinstance(workspace, torch.Tensor) else None))
    workspace = _workspace(workspace, bf16_gemm_workspace_size(M, N, K) if workspace is None else 0, a.device)
    rc = lib().bf16_gemm_packed(_ptr(a), _ptr(wp.packed), M, N, K, _ptr(out), _OUT[out.dtype], out.stride(0),
                                _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("bf16_gemm_packed", rc)
    return out
