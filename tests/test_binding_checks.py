"""Host-side argument checks of the Python binding (no GPU needed).

The C ABI receives only pointers and sizes, so the binding must refuse
tensors whose shape, dtype, layout or device disagree with the sizes it
passes: otherwise the kernels would read or write outside them.  Every case
below is refused before the library is called (CPU tensors with the right
shapes reach only the final device check).
"""
import pytest
import torch

from nvfp4_prefill_gemm_amd import binding as nv

u8, bf16, f32 = torch.uint8, torch.bfloat16, torch.float32


def _nv(M, N, K):
    return (torch.zeros(M, K // 2, dtype=u8), torch.zeros(M, K // 16, dtype=u8), torch.ones(1, dtype=f32),
            torch.zeros(N, K // 2, dtype=u8), torch.zeros(N, K // 16, dtype=u8), torch.ones(1, dtype=f32))


def test_nvfp4_gemm_checks():
    ac, asc, aa, wc, wsc, wa = _nv(8, 16, 64)
    with pytest.raises(ValueError, match="disagree on K"):
        nv.nvfp4_gemm(ac, asc, aa, torch.zeros(16, 16, dtype=u8), wsc, wa)
    with pytest.raises(ValueError, match="a_scales"):
        nv.nvfp4_gemm(ac, torch.zeros(8, 2, dtype=u8), aa, wc, wsc, wa)
    with pytest.raises(ValueError, match="w_scales"):
        nv.nvfp4_gemm(ac, asc, aa, wc, torch.zeros(15, 4, dtype=u8), wa)
    with pytest.raises(TypeError, match="a_alpha"):
        nv.nvfp4_gemm(ac, asc, torch.ones(1, dtype=torch.float64), wc, wsc, wa)
    with pytest.raises(ValueError, match="w_alpha"):
        nv.nvfp4_gemm(ac, asc, aa, wc, wsc, torch.ones(0, dtype=f32))
    with pytest.raises(TypeError, match="a_codes"):
        nv.nvfp4_gemm(ac.to(torch.int8), asc, aa, wc, wsc, wa)
    with pytest.raises(ValueError, match="contiguous"):
        nv.nvfp4_gemm(torch.zeros(8, 64, dtype=u8)[:, ::2], asc, aa, wc, wsc, wa)
    with pytest.raises(ValueError, match="multiple of 16"):
        nv.nvfp4_gemm(torch.zeros(8, 4, dtype=u8), torch.zeros(8, 0, dtype=u8), aa,
                      torch.zeros(16, 4, dtype=u8), torch.zeros(16, 0, dtype=u8), wa)
    # outputs: shape, unit column stride, dtype
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_gemm(ac, asc, aa, wc, wsc, wa, out=torch.empty(8, 15, dtype=f32))
    with pytest.raises(ValueError, match="row-major"):
        nv.nvfp4_gemm(ac, asc, aa, wc, wsc, wa, out=torch.empty(16, 8, dtype=f32).t())
    with pytest.raises(TypeError, match="out"):
        nv.nvfp4_gemm(ac, asc, aa, wc, wsc, wa, out=torch.empty(8, 16, dtype=torch.float16))
    # right shapes on the CPU: only the device check is left
    with pytest.raises(ValueError, match="device tensor"):
        nv.nvfp4_gemm(ac, asc, aa, wc, wsc, wa, out=torch.empty(8, 16, dtype=f32))


def test_quant_out_checks():
    ac, asc, aa, wc, wsc, wa = _nv(8, 32, 64)
    ya = torch.ones(1, dtype=f32)
    with pytest.raises(ValueError, match="y_codes"):
        nv.nvfp4_gemm_quant_out(ac, asc, aa, wc, wsc, wa, ya, y_codes=torch.zeros(8, 15, dtype=u8),
                                y_scales=torch.zeros(8, 2, dtype=u8))
    with pytest.raises(ValueError, match="y_scales"):
        nv.nvfp4_gemm_quant_out(ac, asc, aa, wc, wsc, wa, ya, y_codes=torch.zeros(8, 16, dtype=u8),
                                y_scales=torch.zeros(8, 3, dtype=u8))
    with pytest.raises(TypeError, match="y_alpha"):
        nv.nvfp4_gemm_quant_out(ac, asc, aa, wc, wsc, wa, torch.ones(1, dtype=torch.int32))
    ac, asc, aa, wc, wsc, wa = _nv(8, 24, 64)
    with pytest.raises(ValueError, match="multiple of 16"):
        nv.nvfp4_gemm_quant_out(ac, asc, aa, wc, wsc, wa, ya)


def test_quantize_checks():
    x = torch.zeros(4, 64, dtype=bf16)
    with pytest.raises(TypeError, match="x must be"):
        nv.nvfp4_quantize(x.float())
    with pytest.raises(ValueError, match="multiple of 16"):
        nv.nvfp4_quantize(torch.zeros(4, 40, dtype=bf16))
    with pytest.raises(ValueError, match="codes"):
        nv.nvfp4_quantize(x, codes=torch.zeros(4, 31, dtype=u8), scales=torch.zeros(4, 4, dtype=u8),
                          alpha=torch.ones(1, dtype=f32))
    with pytest.raises(ValueError, match="scales"):
        nv.nvfp4_quantize(x, codes=torch.zeros(4, 32, dtype=u8), scales=torch.zeros(3, 4, dtype=u8),
                          alpha=torch.ones(1, dtype=f32))
    with pytest.raises(ValueError, match="row-major"):
        nv.nvfp4_quantize(torch.zeros(64, 4, dtype=bf16).t())
    with pytest.raises(ValueError, match="static_alpha needs alpha"):
        nv.nvfp4_quantize(x, static_alpha=True)
    # a strided row (ld > cols) is allowed; the CPU tensor is refused last
    with pytest.raises(ValueError, match="device tensor"):
        nv.nvfp4_quantize(torch.zeros(4, 96, dtype=bf16)[:, :64], codes=torch.zeros(4, 32, dtype=u8),
                          scales=torch.zeros(4, 4, dtype=u8), alpha=torch.ones(1, dtype=f32),
                          static_alpha=True)


def test_quant_gemm_and_bf16_checks():
    x = torch.zeros(8, 64, dtype=bf16)
    _, _, _, wc, wsc, wa = _nv(8, 16, 64)
    with pytest.raises(ValueError, match="w_codes"):
        nv.nvfp4_quant_gemm(x, torch.zeros(16, 16, dtype=u8), wsc, wa)
    with pytest.raises(ValueError, match="w_scales"):
        nv.nvfp4_quant_gemm(x, wc, torch.zeros(16, 3, dtype=u8), wa)
    with pytest.raises(ValueError, match="shape"):
        nv.nvfp4_quant_gemm(x, wc, wsc, wa, out=torch.empty(8, 8, dtype=bf16))
    with pytest.raises(ValueError, match="device tensor"):
        nv.nvfp4_quant_gemm(x, wc, wsc, wa, a_alpha=torch.ones(1, dtype=f32), static_alpha=True,
                            out=torch.empty(8, 16, dtype=bf16))
    w = torch.zeros(16, 64, dtype=bf16)
    with pytest.raises(ValueError, match="w must have 64 columns"):
        nv.bf16_gemm(x, torch.zeros(16, 32, dtype=bf16))
    with pytest.raises(ValueError, match="contiguous"):
        nv.bf16_gemm(torch.zeros(8, 128, dtype=bf16)[:, :64], w)
    with pytest.raises(ValueError, match="shape"):
        nv.bf16_gemm(x, w, out=torch.empty(16, 8, dtype=f32))
    with pytest.raises(ValueError, match="device tensor"):
        nv.bf16_gemm(x, w, out=torch.empty(8, 16, dtype=f32))


def test_mxfp4_checks():
    ac, wc = torch.zeros(8, 32, dtype=u8), torch.zeros(16, 32, dtype=u8)
    asc, wsc = torch.zeros(8, 2, dtype=u8), torch.zeros(16, 2, dtype=u8)
    with pytest.raises(ValueError, match="a_scales"):
        nv.mxfp4_gemm(ac, torch.zeros(8, 4, dtype=u8), wc, wsc)
    with pytest.raises(ValueError, match="multiple of 32"):
        nv.mxfp4_gemm(torch.zeros(8, 8, dtype=u8), asc, torch.zeros(16, 8, dtype=u8), wsc)
    with pytest.raises(ValueError, match="disagree on K"):
        nv.mxfp4_gemm(ac, asc, torch.zeros(16, 16, dtype=u8), wsc)
    with pytest.raises(ValueError, match="multiple of 32"):
        nv.mxfp4_quantize(torch.zeros(4, 48, dtype=bf16))
    with pytest.raises(ValueError, match="device tensor"):
        nv.mxfp4_gemm(ac, asc, wc, wsc, out=torch.empty(8, 16, dtype=f32))
