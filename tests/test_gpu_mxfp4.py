"""GPU parity of the MXFP4 path (E2M1 + E8M0 per 32; the coarser format of
Mix-Quant Section 3.3) against the oracle: codes and scales bit-exact, GEMM
outputs within the gate of tests/parity.py."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests import parity
from tests.gpu_util import bf16_dev, bf16_out_to_f64, host, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _quant(nv, xb):
    c, s = nv.mxfp4_quantize(bf16_dev(xb))
    return host(c), host(s)


def _same(got, want, what):
    assert np.array_equal(got[1], want[1]), f"{what}: {np.count_nonzero(got[1] != want[1])} scale mismatches"
    assert np.array_equal(got[0], want[0]), f"{what}: {np.count_nonzero(got[0] != want[0])} code mismatches"


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (130, 288), (257, 4096)])
def test_quantize_shapes(nv, oracle_mod, rows, cols):
    g = np.random.default_rng(rows + cols)
    xb = wl.to_bf16_bits(g.standard_t(4.0, size=(rows, cols)).astype(np.float32))
    say("mxfp4 quantize", rows, cols)
    _same(_quant(nv, xb), oracle_mod.mx_quantize(xb), f"{rows}x{cols}")


def test_quantize_special_values(nv, oracle_mod):
    rows = []
    for amax in (1.0, 1.5, 1.75, 1.9375, 2.0 ** -20, 2.0 ** -130, 3.0e38, 0.0):
        r = np.zeros(64, dtype=np.float32)
        r[5] = amax
        r[6] = -amax / 2
        r[7] = -0.0
        r[40] = amax * 0.3
        rows.append(r)
    ties = np.zeros(64, dtype=np.float32)
    ties[0] = 4.0
    ties[1:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    ties[8:15] = -ties[1:8]
    rows.append(ties)
    xb = wl.to_bf16_bits(np.stack(rows))
    say("mxfp4 quantize special values")
    _same(_quant(nv, xb), oracle_mod.mx_quantize(xb), "special")


@pytest.mark.parametrize("layer", [0, 3])
def test_quantize_qwen3_8b_m8192_full(nv, oracle_mod, layer):
    w = wl.WORKLOADS["qwen3_8b_m8192"]
    a, _ = wl.layer_inputs(w, layer)
    say("mxfp4 quantize qwen3-8b m8192", w.linears[layer][0], a.shape)
    _same(_quant(nv, a), oracle_mod.mx_quantize(a), "qwen3-8b")


def _gemm(nv, A, W, od):
    import torch

    dt = torch.float32 if od == "f32" else torch.bfloat16
    y = nv.mxfp4_gemm(u8_dev(A[0]), u8_dev(A[1]), u8_dev(W[0]), u8_dev(W[1]), out_dtype=dt)
    return host(y).astype(np.float64) if od == "f32" else bf16_out_to_f64(y)


def _bf16_rne(y32):
    return wl.bf16_bits_to_f32(wl.to_bf16_bits(y32.astype(np.float32))).astype(np.float64)


def _check(nv, A, W, ref, what):
    y32, y16 = _gemm(nv, A, W, "f32"), _gemm(nv, A, W, "bf16")
    parity.assert_gemm_close(y32, ref, parity.GEMM_TOL_F32, what + " f32")
    parity.assert_gemm_close(y16, ref, parity.GEMM_TOL_BF16, what + " bf16")
    assert np.array_equal(y16, _bf16_rne(y32)), what + ": BF16 output is not the rounded FP32 output"


@pytest.mark.parametrize("M,N,K", [(32, 32, 256), (256, 256, 256), (512, 512, 1024)])
def test_gemm_unit_scales(nv, oracle_mod, M, N, K):
    """All scales 2^0: isolates the FP4 operand layout of the scaled MFMA."""
    g = np.random.default_rng(M + K)
    A = (g.integers(0, 256, size=(M, K // 2), dtype=np.uint8), np.full((M, K // 32), 127, np.uint8))
    W = (g.integers(0, 256, size=(N, K // 2), dtype=np.uint8), np.full((N, K // 32), 127, np.uint8))
    say("mxfp4 gemm unit scales", M, N, K)
    _check(nv, A, W, oracle_mod.mx_gemm(*A, *W), f"unit scales {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 300, 96), (130, 257, 288), (256, 512, 4096), (300, 520, 1056),
                                   # K % 512 != 0: every tile on the register-staged K-256 path
                                   (256, 256, 128), (256, 512, 384), (512, 256, 640), (256, 256, 896),
                                   # interior tiles with K % 512 == 0 take the pipelined path (1, 2, 3 and
                                   # 5 scale groups); the last case mixes it with edge tiles in one launch
                                   (256, 256, 512), (256, 512, 1024), (512, 256, 1536), (512, 768, 2560),
                                   (300, 520, 1536)])
def test_gemm_random_scales(nv, oracle_mod, M, N, K):
    g = np.random.default_rng(M * 3 + N + K)
    A = (g.integers(0, 256, size=(M, K // 2), dtype=np.uint8), g.integers(110, 140, size=(M, K // 32)).astype(np.uint8))
    W = (g.integers(0, 256, size=(N, K // 2), dtype=np.uint8), g.integers(110, 140, size=(N, K // 32)).astype(np.uint8))
    say("mxfp4 gemm random scales", M, N, K)
    _check(nv, A, W, oracle_mod.mx_gemm(*A, *W), f"random scales {M}x{N}x{K}")


def test_gemm_quantized_tiny(nv, oracle_mod):
    w = wl.WORKLOADS["tiny"]
    a, wt = wl.layer_inputs(w, 0)
    A, W = oracle_mod.mx_quantize(a), oracle_mod.mx_quantize(wt)
    say("mxfp4 gemm tiny")
    _check(nv, A, W, oracle_mod.mx_gemm(*A, *W), "tiny")


@pytest.mark.parametrize("layer", range(4))
def test_gemm_qwen3_8b_m8192_sampled(nv, oracle_mod, layer):
    import torch

    w = wl.WORKLOADS["qwen3_8b_m8192"]
    name, K, N = w.linears[layer]
    a, wt = wl.layer_inputs(w, layer)
    A, W = oracle_mod.mx_quantize(a), oracle_mod.mx_quantize(wt)
    say("mxfp4 gemm qwen3-8b m8192", name, (w.M, N, K))
    ac, asc = nv.mxfp4_quantize(bf16_dev(a))
    wc, wsc = nv.mxfp4_quantize(bf16_dev(wt))
    y = nv.mxfp4_gemm(ac, asc, wc, wsc, out_dtype=torch.bfloat16)
    g = np.random.default_rng(50 + layer)
    mi = np.concatenate([g.integers(0, w.M, 4096), [0, w.M - 1]])
    ni = np.concatenate([g.integers(0, N, 4096), [N - 1, 0]])
    ref = oracle_mod.mx_gemm_pairs(*A, *W, mi, ni)
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy()
    parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"mxfp4 {name} sampled")
