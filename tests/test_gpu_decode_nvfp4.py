"""GPU parity of NVFP4 x NVFP4 at decode shapes (M <= 64), the uniform-NVFP4
and FP4-decode variants of Mix-Quant's ablations: nvfp4_gemm routes these to
the split-K decode kernel when K % 32 == 0, and to the tile kernel
otherwise.  Outputs are compared with the oracle's exact
product under the gate of tests/parity.py; the BF16 output must equal the
nearest-even rounding of the same kernel's FP32 output."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests import parity
from tests.gpu_util import bf16_dev, bf16_out_to_f64, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _bf16_rne(y32):
    return wl.bf16_bits_to_f32(wl.to_bf16_bits(y32.astype(np.float32))).astype(np.float64)


def _run(nv, A, W, out_dtype):
    import torch

    def dev(q):
        return u8_dev(q[0]), u8_dev(q[1]), f32_dev([q[2]])

    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    y = nv.nvfp4_gemm(*dev(A), *dev(W), out_dtype=dt)
    return host(y).astype(np.float64) if out_dtype == "f32" else bf16_out_to_f64(y)


def _check(nv, A, W, ref, what):
    y32 = _run(nv, A, W, "f32")
    y16 = _run(nv, A, W, "bf16")
    parity.assert_gemm_close(y32, ref, parity.GEMM_TOL_F32, what + " f32")
    parity.assert_gemm_close(y16, ref, parity.GEMM_TOL_BF16, what + " bf16")
    assert np.array_equal(y16, _bf16_rne(y32)), what + ": BF16 output is not the rounded FP32 output"
    return y32


@pytest.mark.parametrize("M", wl.PHASE_SPLIT_DECODE_M)
def test_decode_nvfp4_qwen3_8b_full(nv, oracle_mod, M):
    """Batch 1/8/64 through all four Qwen3-8B projections: activation
    quantizer (dynamic alpha over the batch) bit-exact, full outputs."""
    for layer, (name, K, N) in enumerate(wl.QWEN3_8B_LINEARS):
        a = wl.activations(M, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 0))
        wt = wl.weights(N, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 1))
        A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
        say("decode nvfp4", name, M, N, K)
        ac, asc, aal = nv.nvfp4_quantize(bf16_dev(a))
        assert np.array_equal(host(ac), A[0]) and np.array_equal(host(asc), A[1]) and host(aal)[0] == A[2]
        _check(nv, A, W, oracle_mod.gemm_exact(*A, *W), f"decode nvfp4 {name} M={M}")


def _random_operand(g, rows, K, lo=0, hi=127):
    codes = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = g.integers(lo, hi, size=(rows, K // 16)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 15, 96), (16, 17, 160), (17, 300, 4128), (33, 64, 288),
                                   (64, 1000, 1056), (63, 31, 12288),
                                   # wide layers: two 16-row weight groups per workgroup, the last partial
                                   (5, 6200, 1056), (60, 6170, 288)])
def test_decode_nvfp4_ragged(nv, oracle_mod, M, N, K):
    """Ragged M/N/K (K not a multiple of the 128-wide chunk, N not a multiple
    of 16, M in every row-group count), random codes and scale codes
    including the E4M3 subnormals and 448."""
    g = np.random.default_rng(M * 131 + N * 7 + K)
    qa, sa = _random_operand(g, M, K)
    qw, sw = _random_operand(g, N, K)
    sa[:, 0] = np.arange(M, dtype=np.uint8) % 8  # zero and subnormal scales
    sw[::3, -1] = 0x7E
    A, W = (qa, sa, np.float32(3.1e-3)), (qw, sw, np.float32(7.6e-3))
    say("decode nvfp4 ragged", M, N, K)
    _check(nv, A, W, oracle_mod.gemm_exact(*A, *W), f"decode ragged {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 33, 128), (2, 1000, 256), (1, 6200, 4096), (2, 4096, 12288), (2, 17, 1024),
                                   (1, 24576, 4096)])
def test_decode_nvfp4_fp4_mfma_form(nv, oracle_mod, M, N, K):
    """Batches of one or two rows with K % 128 == 0 run the weight codes
    through the FP4 MFMA and scale each 16-element block's exact partial sum
    by sigma_A * sigma_W afterwards: random codes, every E4M3 scale code on
    both operands (zero, the subnormals, 448), one- and two-group strips."""
    g = np.random.default_rng(M * 7 + N * 3 + K)
    qa, sa = _random_operand(g, M, K)
    qw, sw = _random_operand(g, N, K)
    sa[:] = (np.arange(sa.size, dtype=np.int64).reshape(sa.shape) * 5 % 127).astype(np.uint8)
    sw[::7, :] = (np.arange(K // 16) % 8).astype(np.uint8)[None, :]  # rows of zero and subnormal scales
    sw[1::5, ::3] = 0x7E
    A, W = (qa, sa, np.float32(0.37)), (qw, sw, np.float32(2.0 ** -7))
    say("decode nvfp4 fp4-mfma form", M, N, K)
    _check(nv, A, W, oracle_mod.gemm_exact(*A, *W), f"decode fp4 form {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 300, 48), (8, 64, 80), (64, 40, 4112)])
def test_decode_nvfp4_k_not_multiple_of_32(nv, oracle_mod, M, N, K):
    """K % 32 != 0 takes the tile kernel; results still match the oracle."""
    g = np.random.default_rng(K + N)
    A = (*_random_operand(g, M, K, 100, 127), np.float32(1.0))
    W = (*_random_operand(g, N, K, 100, 127), np.float32(0.5))
    say("decode nvfp4 K%32 != 0", M, N, K)
    _check(nv, A, W, oracle_mod.gemm_exact(*A, *W), f"decode K%32 {M}x{N}x{K}")


def test_decode_kernel_agrees_with_tile_kernel(nv, oracle_mod):
    """The same 8 activation rows through the decode kernel (M = 8) and, as
    the first rows of a 65-row problem, through the tile kernel: both within
    the gate of the exact product, and within twice the gate of each other."""
    g = np.random.default_rng(5)
    N, K = 520, 4096
    A65 = (*_random_operand(g, 65, K, 110, 127), np.float32(0.01))
    W = (*_random_operand(g, N, K, 110, 127), np.float32(0.02))
    A8 = (A65[0][:8].copy(), A65[1][:8].copy(), A65[2])
    ref65 = oracle_mod.gemm_exact(*A65, *W)
    say("decode nvfp4 vs tile kernel", N, K)
    y_dec = _check(nv, A8, W, ref65[:8], "decode kernel M=8")
    y_tile = _check(nv, A65, W, ref65, "tile kernel M=65")[:8]
    assert parity.floored_rel_err(y_dec, y_tile) <= 2 * parity.GEMM_TOL_F32


@pytest.mark.parametrize("M,N,K,ld_pad", [(1, 6144, 4096, 0), (1, 4096, 12288, 0), (2, 300, 4128, 8),
                                          (8, 24576, 4096, 0), (13, 17, 96, 24), (16, 1000, 1056, 0),
                                          (16, 64, 12288, 0), (1, 520, 65536, 0), (2, 64, 98304, 0),
                                          (2, 24576, 4096, 16),
                                          # two 16-row weight groups per workgroup, the last one partial
                                          (3, 6200, 1056, 0), (1, 16400, 512, 8), (2, 6200, 12288, 0),
                                          # batch 3-6 on layers up to 8192 columns with M * K <= 32768
                                          # (in-kernel), and just past each limit (quantized once,
                                          # into the packed block layout when K % 128 == 0)
                                          (6, 6144, 4096, 0), (4, 4096, 4096, 8), (5, 8192, 4096, 0),
                                          (6, 8200, 4096, 0), (6, 520, 5472, 0), (6, 4096, 4128, 0),
                                          (7, 6144, 4096, 0), (8, 6144, 4096, 0), (8, 4096, 4096, 8)])
def test_fused_decode_equals_quantize_then_gemm(nv, oracle_mod, M, N, K, ld_pad):
    """nvfp4_quant_gemm at decode sizes: M <= 2 with M * K <= 196608, and
    M <= 6 with N <= 8192 and M * K <= 32768, quantize the batch inside the
    decode kernel (the batch held in registers when it fits, else read
    twice); other batches quantize once into the workspace.  Either way
    alpha, and the output in FP32 and BF16, equal nvfp4_quantize followed by
    nvfp4_gemm bit for bit (dynamic and static
    alpha, strided x, the size limit itself); both within the gate of the
    oracle's exact product."""
    import torch

    g = np.random.default_rng(M * 17 + N + K)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    ref = oracle_mod.gemm_exact(*A, *W)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    xfull = torch.zeros((M, K + ld_pad), dtype=torch.bfloat16, device="cuda")
    xfull[:, :K] = bf16_dev(a)
    x = xfull[:, :K]
    say("fused decode vs quantize+gemm", M, N, K, ld_pad)
    for od in (torch.float32, torch.bfloat16):
        ac, asc, aal = nv.nvfp4_quantize(x)
        y_unf = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=od)
        y_fus, alpha = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=od)
        assert host(alpha)[0] == host(aal)[0] == A[2]
        assert torch.equal(y_fus, y_unf), f"fused decode differs from quantize + gemm ({od})"
        y_st, _ = nv.nvfp4_quant_gemm(x, wc, wsc, wal, a_alpha=f32_dev([A[2]]), static_alpha=True, out_dtype=od)
        assert torch.equal(y_st, y_fus)
        tol = parity.GEMM_TOL_F32 if od == torch.float32 else parity.GEMM_TOL_BF16
        parity.assert_gemm_close(y_fus.float().cpu().numpy(), ref, tol, f"fused decode {M}x{N}x{K}")


def test_fused_decode_zero_batch_and_zero_rows(nv, oracle_mod):
    """An all-zero batch gives alpha 0 and a zero output; a batch whose rows
    are partly zero matches the oracle."""
    import torch

    K, N = 256, 64
    wt = wl.weights(N, K, np.random.default_rng(1))
    W = oracle_mod.quantize(wt)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    say("fused decode zero batch")
    y, alpha = nv.nvfp4_quant_gemm(torch.zeros((3, K), dtype=torch.bfloat16, device="cuda"), wc, wsc, wal,
                                   out_dtype=torch.float32)
    assert host(alpha)[0] == 0.0 and not host(y).any()
    a = wl.activations(5, K, np.random.default_rng(2))
    a[1] = 0
    a[3] = 0x8000  # -0.0
    A = oracle_mod.quantize(a)
    y, alpha = nv.nvfp4_quant_gemm(bf16_dev(a), wc, wsc, wal, out_dtype=torch.float32)
    assert host(alpha)[0] == A[2]
    parity.assert_gemm_close(host(y), oracle_mod.gemm_exact(*A, *W), parity.GEMM_TOL_F32, "partly zero batch")


def test_fused_past_decode_limit_within_gate(nv, oracle_mod):
    """M <= 16 with M * K > 196608: with its full workspace nvfp4_quant_gemm
    quantizes into it and runs the decode GEMM (equal to quantize + gemm bit
    for bit); with only the amax partials the tile kernel quantizes in its
    staging and sums in another order.  Both within the gate."""
    import torch

    M, N, K = 16, 96, 12320
    g = np.random.default_rng(77)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    x = bf16_dev(a)
    ref = oracle_mod.gemm_exact(*A, *W)
    say("fused past decode limit", M, N, K)
    y, alpha = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=torch.float32)
    assert host(alpha)[0] == A[2]
    ac, asc, aal = nv.nvfp4_quantize(x)
    assert torch.equal(y, nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.float32))
    parity.assert_gemm_close(host(y), ref, parity.GEMM_TOL_F32, "quantize into workspace M=16")
    small = torch.empty(max(nv.quantize_workspace_size(M, K), 16), dtype=torch.uint8, device="cuda")
    y2, alpha2 = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=torch.float32, workspace=small)
    assert host(alpha2)[0] == A[2]
    parity.assert_gemm_close(host(y2), ref, parity.GEMM_TOL_F32, "fused tile M=16")


@pytest.mark.parametrize("M,N,K", [(17, 300, 4128), (32, 4096, 4096), (33, 520, 12288), (64, 6144, 4096),
                                   (64, 4096, 12288), (48, 6200, 12320), (64, 24576, 512)])
def test_decode_split_k_vs_unsplit(nv, oracle_mod, M, N, K):
    """Batches above 16 split K over workgroups when given the workspace
    (partial tiles summed in slice order by a second kernel); without it the
    same kernels run unsplit.  NVFP4 and BF16: both ways within the gate of
    the exact product, BF16 output equal to the rounded FP32 output, and
    nvfp4_quant_gemm equal to quantize + gemm bit for bit."""
    import torch

    g = np.random.default_rng(M * 3 + N + K)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    x = bf16_dev(a)
    ac, asc, aal = nv.nvfp4_quantize(x)
    ref = oracle_mod.gemm_exact(*A, *W)
    ref_bf = oracle_mod.bf16_gemm(a, wt)
    say("decode split-K", M, N, K, "nvfp4 ws", nv.gemm_workspace_size(M, N, K),
        "bf16 ws", nv.bf16_gemm_workspace_size(M, N, K))
    for ws in (None, False):
        y32 = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.float32, workspace=ws)
        y16 = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.bfloat16, workspace=ws)
        parity.assert_gemm_close(host(y32), ref, parity.GEMM_TOL_F32, f"nvfp4 {M}x{N}x{K} ws={ws}")
        assert np.array_equal(bf16_out_to_f64(y16), _bf16_rne(host(y32))), "BF16 output is not the rounded FP32"
        if ws is None:
            yq, _ = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=torch.float32)
            assert torch.equal(yq, y32), "nvfp4_quant_gemm differs from quantize + gemm"
        b32 = nv.bf16_gemm(x, bf16_dev(wt), out_dtype=torch.float32, workspace=ws)
        b16 = nv.bf16_gemm(x, bf16_dev(wt), out_dtype=torch.bfloat16, workspace=ws)
        parity.assert_gemm_close(host(b32), ref_bf, parity.GEMM_TOL_F32, f"bf16 {M}x{N}x{K} ws={ws}")
        assert np.array_equal(bf16_out_to_f64(b16), _bf16_rne(host(b32))), "BF16 output is not the rounded FP32"
