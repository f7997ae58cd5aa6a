"""GPU parity of the 256 x 256 tile kernels off their interior fast paths.

Prefill token counts are arbitrary, so the benchmarked 8-wave tile must be
right where a tile crosses the M or N edge (its loads read zeros past the
edge and the epilogue checks rows and columns), where K is not a multiple of
64 (every access checked), and on interior tiles whose K is a multiple of 64
but not of 256 (the block scales fetched per K step, not per group of four).
Each case launches at least 256 output tiles, so the 256 x 256 tile runs,
and is checked on seeded samples of output positions, weighted towards the
last row and column tiles, against the oracle's exact product; the NVFP4
activation codes are compared with the oracle's in full.
"""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests import parity
from tests.gpu_util import bf16_dev, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _pairs(M, N, n, seed):
    """n positions anywhere, n in the last 256-row tile, n in the last
    256-column tile, and the four corners."""
    g = np.random.default_rng(seed)
    lo_m, lo_n = max(0, M - M % 256 if M % 256 else M - 256), max(0, N - N % 256 if N % 256 else N - 256)
    mi = np.concatenate([g.integers(0, M, n), g.integers(lo_m, M, n), g.integers(0, M, n), [0, 0, M - 1, M - 1]])
    ni = np.concatenate([g.integers(0, N, n), g.integers(0, N, n), g.integers(lo_n, N, n), [0, N - 1, 0, N - 1]])
    return mi, ni


def _at(y, mi, ni):
    import torch

    return y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy().astype(np.float64)


def _bf16_rne(y32):
    return wl.bf16_bits_to_f32(wl.to_bf16_bits(y32.astype(np.float32))).astype(np.float64)


def _inputs(M, N, K, seed):
    g = np.random.default_rng(seed)
    return wl.activations(M, K, g), wl.weights(N, K, g)


# (M, N, K): 8000 x 6144 -- edge tiles in M (8000 = 31 * 256 + 64), 768 tiles;
# 4000 x 4100 x 4112 -- edge tiles in M and N and a K tail (4112 % 64 = 16);
# 4096 x 4096 x 576 -- interior tiles, K % 64 == 0, K % 256 != 0
SHAPES = [(8000, 6144, 4096), (4000, 4100, 4112), (4096, 4096, 576)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_nvfp4_gemm_edge_modes(nv, oracle_mod, M, N, K):
    """nvfp4_quantize + nvfp4_gemm (FP32 and BF16 output) and nvfp4_quant_gemm
    with both of its workspace routes, which must equal quantize + GEMM bit
    for bit."""
    import torch

    a, wt = _inputs(M, N, K, M * 31 + N * 7 + K)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("edge tiles nvfp4 gemm", M, N, K)
    x = bf16_dev(a)
    ac, asc, aal = nv.nvfp4_quantize(x)
    assert host(aal)[0] == A[2]
    assert np.array_equal(host(asc), A[1]) and np.array_equal(host(ac), A[0])
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    y32 = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.float32)
    y16 = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.bfloat16)
    mi, ni = _pairs(M, N, 1400, M + N + K)
    ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    got32, got16 = _at(y32, mi, ni), _at(y16, mi, ni)
    parity.assert_gemm_close(got32, ref, parity.GEMM_TOL_F32, f"{M}x{N}x{K} f32 sampled")
    parity.assert_gemm_close(got16, ref, parity.GEMM_TOL_BF16, f"{M}x{N}x{K} bf16 sampled")
    assert np.array_equal(got16, _bf16_rne(got32)), "BF16 output is not the rounded FP32 output"
    small = torch.empty(max(nv.quantize_workspace_size(M, K), 16), dtype=torch.uint8, device="cuda")
    for ws in (None, small):
        say("edge tiles nvfp4 quant_gemm", M, N, K, "full workspace" if ws is None else "prologue")
        yf, alpha = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=torch.bfloat16, workspace=ws)
        assert host(alpha)[0] == A[2]
        assert torch.equal(yf, y16), "nvfp4_quant_gemm must equal nvfp4_quantize + nvfp4_gemm"


@pytest.mark.parametrize("M,N,K", [(8000, 6144, 4096), (4000, 4100, 4104)])
def test_bf16_gemm_edge_modes(nv, oracle_mod, M, N, K):
    """The BF16 tile kernel over M and N edges (8000 x 6144) and with a K tail
    (4104 % 64 = 8)."""
    import torch

    a, wt = _inputs(M, N, K, M + N * 5 + K)
    say("edge tiles bf16 gemm", M, N, K)
    xa, xw = bf16_dev(a), bf16_dev(wt)
    y32 = nv.bf16_gemm(xa, xw, out_dtype=torch.float32)
    y16 = nv.bf16_gemm(xa, xw, out_dtype=torch.bfloat16)
    mi, ni = _pairs(M, N, 1400, 3 * M + N)
    ref = oracle_mod.bf16_gemm_pairs(a, wt, mi, ni)
    got32, got16 = _at(y32, mi, ni), _at(y16, mi, ni)
    parity.assert_gemm_close(got32, ref, parity.GEMM_TOL_F32, f"bf16 {M}x{N}x{K} f32 sampled")
    parity.assert_gemm_close(got16, ref, parity.GEMM_TOL_BF16, f"bf16 {M}x{N}x{K} bf16 sampled")
    assert np.array_equal(got16, _bf16_rne(got32)), "BF16 output is not the rounded FP32 output"


def test_nvfp4_gemm_small_interior_k320(nv, oracle_mod):
    """One interior tile (the 128 x 128 tile at this size) with K % 256 != 0,
    every output against the exact product."""
    import torch

    M, N, K = 256, 256, 320
    a, wt = _inputs(M, N, K, 320)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("nvfp4 gemm interior K=320")
    args = (u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]]))
    y32 = host(nv.nvfp4_gemm(*args, out_dtype=torch.float32)).astype(np.float64)
    parity.assert_gemm_close(y32, oracle_mod.gemm_exact(*A, *W), parity.GEMM_TOL_F32, "256x256x320 f32")


@pytest.mark.parametrize("M,N,K", [(8000, 4096, 4096), (4000, 4112, 4112)])
def test_quant_out_edge_modes(nv, oracle_mod, M, N, K):
    """nvfp4_gemm_quant_out over M and N edge tiles and a K tail: codes and
    block scales against the oracle's FP32 quantizer applied to the FP32
    output of the same product (same summation order), every element; that
    FP32 output against the exact product on samples."""
    import torch

    a, wt = _inputs(M, N, K, M * 3 + N + K)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("edge tiles quant_out", M, N, K)
    args = (u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]]))
    y32 = host(nv.nvfp4_gemm(*args, out_dtype=torch.float32))
    mi, ni = _pairs(M, N, 1000, M * N)
    parity.assert_gemm_close(y32[mi, ni].astype(np.float64), oracle_mod.gemm_exact_pairs(*A, *W, mi, ni),
                             parity.GEMM_TOL_F32, f"{M}x{N}x{K} f32 sampled")
    y_alpha = np.float32(0.02)
    yc, ys = nv.nvfp4_gemm_quant_out(*args, f32_dev([y_alpha]))
    want_c, want_s, _ = oracle_mod.quantize_f32(y32, alpha=float(y_alpha))
    got_c, got_s = host(yc), host(ys)
    assert np.array_equal(got_s, want_s), f"{np.count_nonzero(got_s != want_s)} scale mismatches"
    assert np.array_equal(got_c, want_c), f"{np.count_nonzero(got_c != want_c)} code mismatches"
