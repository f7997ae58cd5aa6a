"""GPU parity of nvfp4_gemm_quant_out: the NVFP4 GEMM whose epilogue
quantizes Y for the next layer (Eq. 3 / Eq. 2 with a static output scale),
and of nvfp4_gemm_quant_out_dynamic (the output scale from Y's own amax).

Where floating point decides the codes, both sides decide in the same
precision: the oracle's FP32 quantizer is applied to the FP32 output of the
same product from the tile GEMM (identical per-element summation order), and
codes and scales must match bit for bit.  The FP32 output itself is checked
against the oracle's exact product under the usual gate."""
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


def _tile_fp32(nv, A, W):
    """FP32 output of the tile GEMM for operands A (M rows) and W: below 65
    rows the operand is padded with zero rows so the tile kernel runs."""
    import torch

    M = A[0].shape[0]
    pad = max(0, 65 - M)
    ac = np.concatenate([A[0], np.zeros((pad, A[0].shape[1]), np.uint8)])
    asc = np.concatenate([A[1], np.zeros((pad, A[1].shape[1]), np.uint8)])
    y = nv.nvfp4_gemm(u8_dev(ac), u8_dev(asc), f32_dev([A[2]]), u8_dev(W[0]), u8_dev(W[1]), f32_dev([W[2]]),
                      out_dtype=torch.float32)
    return host(y)[:M]


def _check(nv, oracle_mod, A, W, y_alpha, what, ref=None, pairs=None):
    """ref: the exact product (full); pairs: (mi, ni, exact values there)."""
    y32 = _tile_fp32(nv, A, W)
    if ref is not None:
        parity.assert_gemm_close(y32, ref, parity.GEMM_TOL_F32, what + " fp32")
    if pairs is not None:
        mi, ni, pref = pairs
        parity.assert_gemm_close(y32[mi, ni], pref, parity.GEMM_TOL_F32, what + " fp32 sampled")
    yc, ys = nv.nvfp4_gemm_quant_out(u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]), u8_dev(W[1]),
                                     f32_dev([W[2]]), f32_dev([y_alpha]))
    want_c, want_s, _ = oracle_mod.quantize_f32(y32, alpha=float(y_alpha))
    got_c, got_s = host(yc), host(ys)
    assert np.array_equal(got_s, want_s), f"{what}: {np.count_nonzero(got_s != want_s)} scale mismatches"
    assert np.array_equal(got_c, want_c), f"{what}: {np.count_nonzero(got_c != want_c)} code mismatches"


@pytest.mark.parametrize("M,N,K", [(128, 256, 256), (1, 16, 16), (33, 48, 96), (130, 272, 272), (300, 528, 1024),
                                   (257, 1040, 4096)])
def test_quant_out_shapes(nv, oracle_mod, M, N, K):
    g = np.random.default_rng(M + N * 3 + K * 7)
    a = wl.activations(M, K, g)
    wt = wl.weights(N, K, g)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    ref = oracle_mod.gemm_exact(*A, *W)
    y_alpha = np.float32(np.max(np.abs(ref)) / 2688.0)
    say("gemm quant out", M, N, K)
    _check(nv, oracle_mod, A, W, y_alpha, f"{M}x{N}x{K}", ref)


@pytest.mark.parametrize("scale", [1.0 / 64, 1.0, 64.0, 2.0 ** 20])
def test_quant_out_output_scale_range(nv, oracle_mod, scale):
    """Output scales far below (codes and block scales saturate at 6 and 448)
    and far above (block scales underflow to E4M3 subnormals and zero) the
    calibrated one."""
    M, N, K = 96, 128, 512
    g = np.random.default_rng(11)
    A = oracle_mod.quantize(wl.activations(M, K, g))
    W = oracle_mod.quantize(wl.weights(N, K, g))
    ref = oracle_mod.gemm_exact(*A, *W)
    y_alpha = np.float32(np.max(np.abs(ref)) / 2688.0 * scale)
    say("gemm quant out scale", scale)
    _check(nv, oracle_mod, A, W, y_alpha, f"scale x{scale}")


def test_quant_out_qwen3_8b_o_proj_full(nv, oracle_mod):
    """The O projection of Qwen3-8B at 8192 tokens (8192 x 4096 x 4096), every
    output code and scale."""
    w = wl.WORKLOADS["qwen3_8b_m8192"]
    name, K, N = w.linears[1]
    a, wt = wl.layer_inputs(w, 1)
    say("gemm quant out qwen3-8b", name, (w.M, N, K))
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    ac, asc, aal = nv.nvfp4_quantize(bf16_dev(a))  # the library's quantizer on the way in: bit-exact
    assert host(aal)[0] == A[2] and np.array_equal(host(asc), A[1]) and np.array_equal(host(ac), A[0])
    y_alpha = np.float32(0.02)
    g = np.random.default_rng(5)
    mi = np.concatenate([g.integers(0, w.M, 4096), [0, w.M - 1]])
    ni = np.concatenate([g.integers(0, N, 4096), [N - 1, 0]])
    pref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    _check(nv, oracle_mod, A, W, y_alpha, "qwen3-8b o_proj", pairs=(mi, ni, pref))


def test_quant_out_k_zero_and_errors(nv):
    import torch

    say("gemm quant out K=0 / errors")
    z = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    one = f32_dev([1.0])
    yc = torch.full((4, 8), 0x77, dtype=torch.uint8, device="cuda")
    ys = torch.full((4, 1), 0x77, dtype=torch.uint8, device="cuda")
    w0 = torch.empty((16, 0), dtype=torch.uint8, device="cuda")
    nv.nvfp4_gemm_quant_out(z, z, one, w0, w0, one, one, yc, ys)
    assert not host(yc).any() and not host(ys).any()
    a = torch.zeros((4, 8), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 1), dtype=torch.uint8, device="cuda")
    w = torch.zeros((24, 8), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((24, 1), dtype=torch.uint8, device="cuda")
    # the binding refuses N % 16 != 0 before the call; the C ABI refuses it too
    with pytest.raises(ValueError, match="multiple of 16"):
        nv.nvfp4_gemm_quant_out(a, s, one, w, ws, one, one)
    yc2 = torch.zeros((4, 12), dtype=torch.uint8, device="cuda")
    ys2 = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    rc = nv.lib().nvfp4_gemm_quant_out(nv._ptr(a), nv._ptr(s), nv._ptr(one), nv._ptr(w), nv._ptr(ws), nv._ptr(one),
                                       4, 24, 16, nv._ptr(yc2), nv._ptr(ys2), nv._ptr(one), nv._stream(None))
    assert rc == nv.NVFP4_EINVAL and "multiple of 16" in nv.last_error()


def _check_dynamic(nv, oracle_mod, A, W, what, ref=None, pairs=None):
    """Dynamic output scale: alpha_Y, codes and scales bit-exact against the
    oracle's FP32 quantizer (dynamic alpha) on the tile GEMM's FP32 output."""
    y32 = _tile_fp32(nv, A, W)
    if ref is not None:
        parity.assert_gemm_close(y32, ref, parity.GEMM_TOL_F32, what + " fp32")
    if pairs is not None:
        mi, ni, pref = pairs
        parity.assert_gemm_close(y32[mi, ni], pref, parity.GEMM_TOL_F32, what + " fp32 sampled")
    yc, ys, ya = nv.nvfp4_gemm_quant_out_dynamic(u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]),
                                                 u8_dev(W[1]), f32_dev([W[2]]))
    want_c, want_s, want_a = oracle_mod.quantize_f32(y32)
    assert host(ya)[0] == want_a, f"{what}: alpha {host(ya)[0]!r} != {want_a!r}"
    got_c, got_s = host(yc), host(ys)
    assert np.array_equal(got_s, want_s), f"{what}: {np.count_nonzero(got_s != want_s)} scale mismatches"
    assert np.array_equal(got_c, want_c), f"{what}: {np.count_nonzero(got_c != want_c)} code mismatches"
    return yc, ys, ya


@pytest.mark.parametrize("M,N,K", [(128, 256, 256), (1, 16, 16), (33, 48, 96), (130, 272, 272), (300, 528, 1024),
                                   (257, 1040, 4096), (512, 512, 512)])
def test_quant_out_dynamic_shapes(nv, oracle_mod, M, N, K):
    g = np.random.default_rng(M * 5 + N + K * 3)
    A = oracle_mod.quantize(wl.activations(M, K, g))
    W = oracle_mod.quantize(wl.weights(N, K, g))
    say("gemm quant out dynamic", M, N, K)
    _check_dynamic(nv, oracle_mod, A, W, f"dynamic {M}x{N}x{K}", ref=oracle_mod.gemm_exact(*A, *W))


def test_quant_out_dynamic_matches_static_with_its_alpha(nv, oracle_mod):
    """With the dynamic call's alpha_Y passed as a static scale, the epilogue
    quantizer gives the same codes and scales."""
    M, N, K = 300, 528, 1024
    g = np.random.default_rng(23)
    A = oracle_mod.quantize(wl.activations(M, K, g))
    W = oracle_mod.quantize(wl.weights(N, K, g))
    say("gemm quant out dynamic vs static")
    yc, ys, ya = _check_dynamic(nv, oracle_mod, A, W, "dynamic vs static")
    sc, ss = nv.nvfp4_gemm_quant_out(u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]), u8_dev(W[1]),
                                     f32_dev([W[2]]), ya)
    assert np.array_equal(host(sc), host(yc)) and np.array_equal(host(ss), host(ys))


def test_quant_out_dynamic_qwen3_8b_o_proj_full(nv, oracle_mod):
    """The O projection of Qwen3-8B at 8192 tokens (8192 x 4096 x 4096), every
    output code and scale and the output tensor scale."""
    w = wl.WORKLOADS["qwen3_8b_m8192"]
    name, K, N = w.linears[1]
    a, wt = wl.layer_inputs(w, 1)
    say("gemm quant out dynamic qwen3-8b", name, (w.M, N, K))
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    g = np.random.default_rng(6)
    mi = np.concatenate([g.integers(0, w.M, 4096), [0, w.M - 1]])
    ni = np.concatenate([g.integers(0, N, 4096), [N - 1, 0]])
    pref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    _check_dynamic(nv, oracle_mod, A, W, "dynamic qwen3-8b o_proj", pairs=(mi, ni, pref))


def test_quant_out_dynamic_two_calls_reuse_workspace(nv, oracle_mod):
    """One workspace for two calls in a row (larger, then smaller product):
    the second result does not depend on what the first left behind."""
    import torch

    say("gemm quant out dynamic workspace reuse")
    big = (384, 512, 512)
    ws = torch.empty(nv.gemm_quant_out_dynamic_workspace_size(*big), dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate((big, (65, 64, 256))):
        g = np.random.default_rng(70 + i)
        A = oracle_mod.quantize(wl.activations(M, K, g))
        W = oracle_mod.quantize(wl.weights(N, K, g))
        yc, ys, ya = nv.nvfp4_gemm_quant_out_dynamic(u8_dev(A[0]), u8_dev(A[1]), f32_dev([A[2]]), u8_dev(W[0]),
                                                     u8_dev(W[1]), f32_dev([W[2]]), workspace=ws)
        want_c, want_s, want_a = oracle_mod.quantize_f32(_tile_fp32(nv, A, W))
        assert host(ya)[0] == want_a
        assert np.array_equal(host(ys), want_s) and np.array_equal(host(yc), want_c)


def test_quant_out_dynamic_k_zero(nv):
    import torch

    say("gemm quant out dynamic K=0")
    z = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    w0 = torch.empty((16, 0), dtype=torch.uint8, device="cuda")
    one = f32_dev([1.0])
    yc = torch.full((4, 8), 0x77, dtype=torch.uint8, device="cuda")
    ys = torch.full((4, 1), 0x77, dtype=torch.uint8, device="cuda")
    ya = f32_dev([3.0])
    nv.nvfp4_gemm_quant_out_dynamic(z, z, one, w0, w0, one, yc, ys, ya)
    assert not host(yc).any() and not host(ys).any() and host(ya)[0] == 0.0
