"""GPU parity of the decode-packed NVFP4 weights (nvfp4_decode_pack,
nvfp4_gemm_packed, nvfp4_quant_gemm_packed): the packed bytes against the
layout's definition (tests/decode_pack_ref.py, from include/nvfp4.h); the
packed GEMMs against the row-major entry points bit for bit (the same codes
and scales through the same kernels in the same order), over every decode
plan (batch 1-64, the FP4-MFMA and FP16 forms, fused and quantize-first
routes, split and unsplit K, ragged N); and against the oracle's exact
product under the gate of tests/parity.py."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests import decode_pack_ref, parity
from tests.gpu_util import bf16_dev, f32_dev, host, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _random_operand(g, rows, K, lo=0, hi=127):
    return (g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8),
            g.integers(lo, hi, size=(rows, K // 16)).astype(np.uint8))


@pytest.mark.parametrize("N,K", [(1, 128), (40, 384), (1000, 512), (6144, 4096), (4100, 12288)])
def test_pack_bytes(nv, N, K):
    g = np.random.default_rng(N + K)
    codes, scales = _random_operand(g, N, K)
    say("decode pack", N, K)
    wp = nv.nvfp4_decode_pack(u8_dev(codes), u8_dev(scales), f32_dev([0.5]))
    assert wp.n == N and wp.k == K
    assert np.array_equal(host(wp.packed), decode_pack_ref.pack(codes, scales))


@pytest.mark.parametrize("M,N,K", [(1, 33, 128), (2, 1000, 512), (3, 1000, 512), (8, 6144, 4096),
                                   (16, 4100, 1024), (17, 300, 4096), (33, 520, 12288), (64, 6144, 4096),
                                   (64, 24576, 4096), (64, 4096, 12288), (1, 24576, 4096), (2, 4096, 12288)])
def test_gemm_packed_equals_row_major(nv, oracle_mod, M, N, K):
    """nvfp4_gemm_packed == nvfp4_gemm bit for bit (FP32 and BF16 out, with
    the split-K workspace and without); the FP32 output within the gate of
    the exact product."""
    import torch

    g = np.random.default_rng(M * 31 + N + K)
    qa, sa = _random_operand(g, M, K, 90, 127)
    qw, sw = _random_operand(g, N, K, 90, 127)
    sw[::5, 1] = 0  # zero and subnormal scales
    sw[1::7, 2] = 3
    A, W = (qa, sa, np.float32(0.02)), (qw, sw, np.float32(0.003))
    ac, asc, aal = u8_dev(qa), u8_dev(sa), f32_dev([A[2]])
    wc, wsc, wal = u8_dev(qw), u8_dev(sw), f32_dev([W[2]])
    say("gemm packed vs row-major", M, N, K)
    wp = nv.nvfp4_decode_pack(wc, wsc, wal)
    for ws in (None, False):
        for od in (torch.float32, torch.bfloat16):
            y_rm = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=od, workspace=ws)
            y_pk = nv.nvfp4_gemm_packed(ac, asc, aal, wp, out_dtype=od, workspace=ws)
            assert torch.equal(y_pk, y_rm), f"packed differs from row-major ({od}, workspace {ws})"
    if M * N * K <= 64 * 6144 * 4096:
        ref = oracle_mod.gemm_exact(*A, *W)
        y = nv.nvfp4_gemm_packed(ac, asc, aal, wp, out_dtype=torch.float32)
        parity.assert_gemm_close(host(y), ref, parity.GEMM_TOL_F32, f"packed {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 6144, 4096), (1, 24576, 4096), (1, 4096, 12288), (2, 4096, 12288),
                                   (4, 4096, 4096), (8, 6144, 4096), (8, 24576, 4096), (8, 4096, 12288),
                                   (16, 1000, 512), (33, 6144, 4096), (64, 24576, 4096), (64, 4096, 12288),
                                   (2, 6200, 1024)])
def test_quant_gemm_packed_equals_row_major(nv, oracle_mod, M, N, K):
    """nvfp4_quant_gemm_packed == nvfp4_quant_gemm bit for bit, alpha
    included (dynamic and static alpha, FP32 and BF16 out): the fused decode
    kernel's batches and the quantize-first ones."""
    import torch

    g = np.random.default_rng(M * 7 + N * 3 + K)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    W = oracle_mod.quantize(wt)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    x = bf16_dev(a)
    say("quant gemm packed vs row-major", M, N, K)
    wp = nv.nvfp4_decode_pack(wc, wsc, wal)
    for od in (torch.float32, torch.bfloat16):
        y_rm, al_rm = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=od)
        y_pk, al_pk = nv.nvfp4_quant_gemm_packed(x, wp, out_dtype=od)
        assert host(al_pk)[0] == host(al_rm)[0]
        assert torch.equal(y_pk, y_rm), f"packed differs from row-major ({od})"
        y_st, _ = nv.nvfp4_quant_gemm_packed(x, wp, a_alpha=al_rm.clone(), static_alpha=True, out_dtype=od)
        assert torch.equal(y_st, y_rm)


@pytest.mark.parametrize("M,N,K,ld_pad", [(3, 1000, 128, 0), (7, 6144, 4096, 8), (8, 24576, 4096, 0),
                                          (17, 520, 1152, 0), (33, 6144, 4096, 16), (40, 4096, 12288, 0),
                                          (63, 24576, 4096, 0), (64, 4100, 12288, 8), (64, 16, 128, 0)])
def test_quant_gemm_packed_activation_layout(nv, oracle_mod, M, N, K, ld_pad):
    """Decode batches of 3-64 rows with K % 128 == 0 that nvfp4_quant_gemm
    quantizes into its workspace: the quantizer writes the batch in the decode
    kernel's block layout (ragged last row group, strided x).  Row-major and
    packed weights, dynamic and static alpha, FP32 and BF16 out: equal bit for
    bit to nvfp4_quantize followed by nvfp4_gemm (row-major codes), and within
    the gate of the oracle's exact product."""
    import torch

    g = np.random.default_rng(M * 31 + N * 5 + K)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    wc, wsc, wal = u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]])
    wp = nv.nvfp4_decode_pack(wc, wsc, wal)
    xfull = torch.zeros((M, K + ld_pad), dtype=torch.bfloat16, device="cuda")
    xfull[:, :K] = bf16_dev(a)
    x = xfull[:, :K]
    say("quant gemm packed activation", M, N, K, ld_pad)
    ac, asc, aal = nv.nvfp4_quantize(x)
    assert host(aal)[0] == A[2]
    for od in (torch.float32, torch.bfloat16):
        y_ref = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=od)
        y_rm, al_rm = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=od)
        y_pk, al_pk = nv.nvfp4_quant_gemm_packed(x, wp, out_dtype=od)
        assert host(al_rm)[0] == host(al_pk)[0] == A[2]
        assert torch.equal(y_rm, y_ref), f"quant_gemm differs from quantize + gemm ({od})"
        assert torch.equal(y_pk, y_ref), f"quant_gemm_packed differs from quantize + gemm ({od})"
        y_st, _ = nv.nvfp4_quant_gemm_packed(x, wp, a_alpha=f32_dev([A[2]]), static_alpha=True, out_dtype=od)
        assert torch.equal(y_st, y_ref)
        tol = parity.GEMM_TOL_F32 if od == torch.float32 else parity.GEMM_TOL_BF16
        parity.assert_gemm_close(y_pk.float().cpu().numpy(), oracle_mod.gemm_exact(*A, *W), tol,
                                 f"packed activation {M}x{N}x{K}")


@pytest.mark.parametrize("M", wl.PHASE_SPLIT_DECODE_M)
def test_quant_gemm_packed_qwen3_8b_vs_oracle(nv, oracle_mod, M):
    """Batch 1/8/64 through the Qwen3-8B qkv and down projections on packed
    weights: alpha equal to the oracle's, output within the gate of the
    exact product of the oracle's quantized operands."""
    import torch

    for layer, (name, K, N) in enumerate(wl.QWEN3_8B_LINEARS):
        if name not in ("qkv", "down"):
            continue
        a = wl.activations(M, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 0))
        wt = wl.weights(N, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 1))
        A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
        say("quant gemm packed vs oracle", name, M, N, K)
        wp = nv.nvfp4_decode_pack(u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]]))
        y, alpha = nv.nvfp4_quant_gemm_packed(bf16_dev(a), wp, out_dtype=torch.float32)
        assert host(alpha)[0] == A[2]
        parity.assert_gemm_close(host(y), oracle_mod.gemm_exact(*A, *W), parity.GEMM_TOL_F32,
                                 f"packed decode {name} M={M}")


def test_quant_gemm_packed_workspace_errors(nv):
    """A quantize-first batch without room for the quantized batch is refused
    (the row-major entry point would fall back to the tile kernel, which
    cannot read packed weights)."""
    import torch

    M, N, K = 32, 512, 1024
    wc = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    wsc = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    wp = nv.nvfp4_decode_pack(wc, wsc, f32_dev([1.0]))
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(nv.quantize_workspace_size(M, K) + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_quant_gemm_packed(x, wp, workspace=small)
    assert e.value.code == nv.NVFP4_EWORKSPACE


@pytest.mark.parametrize("N,K", [(1, 32), (40, 96), (1000, 4128), (6144, 4096)])
def test_bf16_pack_bytes(nv, N, K):
    g = np.random.default_rng(N * 3 + K)
    w = g.integers(0, 65536, size=(N, K), dtype=np.uint16)
    say("bf16 decode pack", N, K)
    wp = nv.bf16_decode_pack(bf16_dev(w))
    assert wp.n == N and wp.k == K
    assert np.array_equal(host(wp.packed), decode_pack_ref.pack_bf16(w))


@pytest.mark.parametrize("M,N,K", [(1, 33, 32), (1, 6144, 4096), (1, 4096, 12288), (2, 1000, 4128), (8, 6144, 4096),
                                   (8, 4096, 4096), (16, 300, 1056), (17, 300, 4096), (33, 520, 12288),
                                   (64, 24576, 4096), (64, 4096, 12288), (64, 6144, 4096), (48, 6200, 4160)])
def test_bf16_gemm_packed_equals_row_major(nv, oracle_mod, M, N, K):
    """bf16_gemm_packed == bf16_gemm bit for bit (FP32 and BF16 out, with the
    split-K workspace and without); the FP32 output within the gate of the
    oracle's BF16 product."""
    import torch

    g = np.random.default_rng(M * 11 + N + K)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    x, w = bf16_dev(a), bf16_dev(wt)
    say("bf16 gemm packed vs row-major", M, N, K)
    wp = nv.bf16_decode_pack(w)
    for ws in (None, False):
        for od in (torch.float32, torch.bfloat16):
            y_rm = nv.bf16_gemm(x, w, out_dtype=od, workspace=ws)
            y_pk = nv.bf16_gemm_packed(x, wp, out_dtype=od, workspace=ws)
            assert torch.equal(y_pk, y_rm), f"packed differs from row-major ({od}, workspace {ws})"
    if M * N * K <= 64 * 6144 * 4096:
        y = nv.bf16_gemm_packed(x, wp, out_dtype=torch.float32)
        parity.assert_gemm_close(host(y), oracle_mod.bf16_gemm(a, wt), parity.GEMM_TOL_F32,
                                 f"bf16 packed {M}x{N}x{K}")
