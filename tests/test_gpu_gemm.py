"""GPU parity of the GEMMs against the oracle.

NVFP4 GEMM, fused quantize-in-GEMM and BF16 GEMM outputs are compared element
by element with the oracle's exact product (and the literal FP32 product on
the tiny case) under the floored relative-error gate of tests/parity.py:
1e-3 for FP32 output, 1e-3 + 2^-8 (BF16 output rounding) for BF16 output.  Full-size layers are
checked on seeded samples of output positions computed one by one.
"""
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


def _dev_operand(q):
    codes, scales, alpha = q
    return u8_dev(codes), u8_dev(scales), f32_dev([alpha])


def _gemm(nv, A, W, out_dtype):
    import torch

    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    y = nv.nvfp4_gemm(*_dev_operand(A), *_dev_operand(W), out_dtype=dt)
    return host(y).astype(np.float64) if out_dtype == "f32" else bf16_out_to_f64(y)


def _tol(out_dtype):
    return parity.GEMM_TOL_F32 if out_dtype == "f32" else parity.GEMM_TOL_BF16


def _bf16_rne(y32: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even BF16 value (as float64)."""
    return wl.bf16_bits_to_f32(wl.to_bf16_bits(y32.astype(np.float32))).astype(np.float64)


def _check_both_outputs(y32, y16, ref, what):
    """FP32 output within the gate; BF16 output equal to the nearest-even
    rounding of the FP32 output of the same kernel (same accumulation)."""
    parity.assert_gemm_close(y32, ref, parity.GEMM_TOL_F32, what + " f32")
    parity.assert_gemm_close(y16, ref, parity.GEMM_TOL_BF16, what + " bf16")
    assert np.array_equal(y16, _bf16_rne(y32)), what + ": BF16 output is not the rounded FP32 output"


def test_tiny_config_full(nv, oracle_mod):
    w = wl.WORKLOADS["tiny"]
    a, wt = wl.layer_inputs(w, 0)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    ref = oracle_mod.gemm_exact(*A, *W)
    ref32 = oracle_mod.gemm_fp32(*A, *W)
    say("nvfp4 gemm tiny")
    y32, y16 = _gemm(nv, A, W, "f32"), _gemm(nv, A, W, "bf16")
    _check_both_outputs(y32, y16, ref, "tiny vs exact")
    parity.assert_gemm_close(y32, ref32, parity.GEMM_TOL_F32, "tiny f32 vs fp32 literal")


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (1, 300, 48), (127, 129, 80), (130, 257, 272), (300, 520, 1024),
                                   (64, 64, 4096), (256, 128, 16),
                                   # interior tiles with K % 256 == 0 fetch block scales per group of
                                   # four K steps: one, two and three groups, and mixed with edge tiles
                                   (256, 256, 256), (384, 256, 512), (128, 128, 768), (300, 520, 768)])
def test_ragged_shapes(nv, oracle_mod, M, N, K):
    g = np.random.default_rng(M * 7 + N * 13 + K)
    a = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    wt = wl.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * 0.02)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    ref = oracle_mod.gemm_exact(*A, *W)
    say("nvfp4 gemm ragged", M, N, K)
    _check_both_outputs(_gemm(nv, A, W, "f32"), _gemm(nv, A, W, "bf16"), ref, f"{M}x{N}x{K}")


def test_extreme_scale_codes(nv, oracle_mod):
    """Random E2M1 codes with every E4M3 scale code that can occur: the seven
    subnormals (m * 2^-9), 448, and zero blocks; tiny and large tensor scales."""
    g = np.random.default_rng(31)
    M, N, K = 160, 288, 512
    qa = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qw = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa = g.integers(0, 127, size=(M, K // 16)).astype(np.uint8)
    sw = g.integers(0, 127, size=(N, K // 16)).astype(np.uint8)
    sa[:, :8] = np.arange(8, dtype=np.uint8)[None, :]  # 0 and the subnormals
    sw[:, 8:16] = np.arange(8, dtype=np.uint8)[None, :]
    sa[::3, 20] = 0x7E
    sw[::5, 20] = 0x7E
    for aa, aw in ((1.0, 1.0), (np.float32(3.1e-3), np.float32(7.6e-6)), (np.float32(2.0 ** -20), np.float32(1024.0))):
        A, W = (qa, sa, np.float32(aa)), (qw, sw, np.float32(aw))
        ref = oracle_mod.gemm_exact(*A, *W)
        say("nvfp4 gemm extreme scale codes", aa, aw)
        _check_both_outputs(_gemm(nv, A, W, "f32"), _gemm(nv, A, W, "bf16"), ref, f"extreme scales {aa},{aw}")


def test_k_zero_and_empty(nv):
    import torch

    say("nvfp4 gemm K=0 / M=0")
    z = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    s = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    one = f32_dev([1.0])
    y = torch.full((4, 4), 7.0, device="cuda")
    nv.nvfp4_gemm(z, s, one, z, s, one, out=y)
    assert host(y).tolist() == [[0.0] * 4] * 4
    e = torch.empty((0, 8), dtype=torch.uint8, device="cuda")
    es = torch.empty((0, 1), dtype=torch.uint8, device="cuda")
    w = torch.zeros((4, 8), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((4, 1), dtype=torch.uint8, device="cuda")
    out = nv.nvfp4_gemm(e, es, one, w, ws, one, out_dtype=torch.float32)
    assert tuple(out.shape) == (0, 4)


@pytest.mark.parametrize("M,N,K", [(512, 512, 1024), (4096, 4096, 512)])
def test_scales_four_byte_aligned(nv, oracle_mod, M, N, K):
    """Scale arrays at the documented minimum alignment (4 bytes, not 8):
    interior tiles with K % 256 == 0 fetch a row's block scales 8 bytes at a
    time, so these loads are 4-byte aligned here.  The 128 x 128 tile and the
    8-wave 256 x 256 tile; same result as 16-byte aligned scales, and the
    oracle on sampled outputs."""
    import torch

    g = np.random.default_rng(M + 3 * K)
    qa = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qw = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa = g.integers(0, 127, size=(M, K // 16)).astype(np.uint8)
    sw = g.integers(0, 127, size=(N, K // 16)).astype(np.uint8)
    one = f32_dev([1.0])

    def off4(a):
        buf = torch.zeros(a.size + 4, dtype=torch.uint8, device="cuda")
        v = buf[4:].view(a.shape)
        v.copy_(torch.from_numpy(a).cuda())
        assert v.data_ptr() % 8 == 4
        return v

    say("nvfp4 gemm 4-byte aligned scales", M, N, K)
    y_al = nv.nvfp4_gemm(u8_dev(qa), u8_dev(sa), one, u8_dev(qw), u8_dev(sw), one, out_dtype=torch.float32)
    y_off = nv.nvfp4_gemm(u8_dev(qa), off4(sa), one, u8_dev(qw), off4(sw), one, out_dtype=torch.float32)
    assert torch.equal(y_off, y_al), "4-byte aligned scales change the result"
    mi, ni = _sample_pairs(M, N, 2000, M + K)
    ref = oracle_mod.gemm_exact_pairs(qa, sa, np.float32(1.0), qw, sw, np.float32(1.0), mi, ni)
    got = y_off[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy().astype(np.float64)
    parity.assert_gemm_close(got, ref, parity.GEMM_TOL_F32, f"4-byte aligned scales {M}x{N}x{K}")


def _sample_pairs(M, N, n, seed):
    g = np.random.default_rng(seed)
    mi = np.concatenate([g.integers(0, M, n), [0, M - 1, M - 1, 0]])
    ni = np.concatenate([g.integers(0, N, n), [0, N - 1, 0, N - 1]])
    return mi, ni


@pytest.mark.parametrize("layer", range(4))
def test_qwen3_8b_m8192_sampled(nv, oracle_mod, layer):
    """Full-size Qwen3-8B prefill linear at 8192 tokens, BF16 output as timed by
    the benchmark; 4096 sampled outputs against the exact oracle."""
    import torch

    w = wl.WORKLOADS["qwen3_8b_m8192"]
    name, K, N = w.linears[layer]
    a, wt = wl.layer_inputs(w, layer)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("nvfp4 gemm qwen3-8b m8192", name, (w.M, N, K))
    x = bf16_dev(a)
    ac, asc, aal = nv.nvfp4_quantize(x)
    wc, wsc, wal = _dev_operand(W)
    y = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.bfloat16)
    y32 = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.float32)
    mi, ni = _sample_pairs(w.M, N, 4096, layer)
    ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    idx = (torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda())
    got = y[idx].float().cpu().numpy().astype(np.float64)
    got32 = y32[idx].cpu().numpy().astype(np.float64)
    parity.assert_gemm_close(got32, ref, parity.GEMM_TOL_F32, f"{name} sampled f32")
    parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"{name} sampled bf16")
    assert np.array_equal(got, _bf16_rne(got32)), f"{name}: BF16 output is not the rounded FP32 output"


def _small_workspace(nv, M, K):
    """A workspace that holds only the dynamic alpha's partials: nvfp4_quant_gemm
    then quantizes inside the tile kernel's operand staging."""
    import torch

    return torch.empty(max(nv.quantize_workspace_size(M, K), 16), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("M,N,K", [(128, 256, 256), (200, 136, 528), (1024, 512, 4096),
                                   # edge tiles, K tail, and the 256 x 256 tile with edges
                                   (300, 520, 784), (4000, 4100, 4112)])
def test_fused_equals_unfused_and_oracle(nv, oracle_mod, M, N, K):
    """nvfp4_quant_gemm, both ways: with its full workspace (quantize into the
    workspace, then the NVFP4 GEMM) and with only the amax partials (the tile
    kernel quantizes in its operand staging): alpha and outputs equal
    nvfp4_quantize followed by nvfp4_gemm bit for bit, dynamic and static."""
    import torch

    g = np.random.default_rng(M + N + K)
    a = wl.to_bf16_bits(g.standard_t(4.0, size=(M, K)).astype(np.float32))
    wt = wl.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * 0.02)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    wc, wsc, wal = _dev_operand(W)
    x = bf16_dev(a)
    for od in (torch.float32, torch.bfloat16):
        ac, asc, aal = nv.nvfp4_quantize(x)
        y_unf = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=od)
        for full in (True, False):
            say("fused vs unfused", M, N, K, od, "full workspace" if full else "prologue")
            ws = None if full else _small_workspace(nv, M, K)
            y_fus, alpha = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=od, workspace=ws)
            assert host(alpha)[0] == host(aal)[0] == A[2]
            assert torch.equal(y_unf, y_fus), "fused and unfused paths must agree bit for bit"
            ys, _ = nv.nvfp4_quant_gemm(x, wc, wsc, wal, a_alpha=f32_dev([A[2]]), static_alpha=True, out_dtype=od,
                                        workspace=ws)
            assert torch.equal(ys, y_fus)
    if M * N <= 1 << 20:
        ref = oracle_mod.gemm_exact(*A, *W)
        parity.assert_gemm_close(y_fus.float().cpu().numpy(), ref, parity.GEMM_TOL_BF16, f"fused {M}x{N}x{K}")
    else:
        mi, ni = _sample_pairs(M, N, 2000, M + N)
        ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
        got = y_fus[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy()
        parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"fused {M}x{N}x{K} sampled")


def test_fused_student_t_long_prefill_sampled(nv, oracle_mod):
    """Fused path on the long agentic prefill: 32768 tokens of Student-t(4)
    activations into the Qwen3-8B QKV projection, sampled outputs."""
    import torch

    w = wl.WORKLOADS["qwen3_8b_m32768_t4"]
    name, K, N = w.linears[0]
    a, wt = wl.layer_inputs(w, 0)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("fused gemm student-t m32768", name, (w.M, N, K))
    wc, wsc, wal = _dev_operand(W)
    x = bf16_dev(a)
    mi, ni = _sample_pairs(w.M, N, 4096, 99)
    ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    for full in (True, False):
        y, alpha = nv.nvfp4_quant_gemm(x, wc, wsc, wal, out_dtype=torch.bfloat16,
                                       workspace=None if full else _small_workspace(nv, w.M, K))
        assert host(alpha)[0] == A[2]
        got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy()
        parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"fused student-t sampled (full ws {full})")


# ------------------------------------------------------------------ BF16 path
def _bf16(nv, a, wt, od):
    import torch

    dt = torch.float32 if od == "f32" else torch.bfloat16
    y = nv.bf16_gemm(bf16_dev(a), bf16_dev(wt), out_dtype=dt)
    return host(y).astype(np.float64) if od == "f32" else bf16_out_to_f64(y)


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (1, 4096, 4096), (8, 300, 136), (17, 64, 512), (64, 1000, 1032),
                                   (65, 129, 264), (300, 520, 1024),
                                   # batch 33-64 on a wide layer: 128-column decode strips, the last one partial
                                   (40, 16400, 520), (64, 16384, 4096)])
def test_bf16_gemm_shapes(nv, oracle_mod, M, N, K):
    g = np.random.default_rng(M * 3 + N + K)
    a = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    wt = wl.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * 0.02)
    ref = oracle_mod.bf16_gemm(a, wt)
    say("bf16 gemm", M, N, K)
    _check_both_outputs(_bf16(nv, a, wt, "f32"), _bf16(nv, a, wt, "bf16"), ref, f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M", wl.PHASE_SPLIT_DECODE_M)
def test_decode_qwen3_8b_full(nv, oracle_mod, M):
    """BF16 decode GEMMs at batch 1/8/64 on the Qwen3-8B projections (full outputs)."""
    for layer, (name, K, N) in enumerate(wl.QWEN3_8B_LINEARS):
        g = wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 0)
        a = wl.activations(M, K, g)
        wt = wl.weights(N, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 1))
        say("decode bf16 gemm", name, M, N, K)
        ref = oracle_mod.bf16_gemm(a, wt)
        parity.assert_gemm_close(_bf16(nv, a, wt, "bf16"), ref, parity.GEMM_TOL_BF16, f"decode {name} M={M}")


@pytest.mark.parametrize("layer", range(4))
def test_bf16_prefill_qwen3_8b_m8192_sampled(nv, oracle_mod, layer):
    import torch

    w = wl.WORKLOADS["qwen3_8b_m8192"]
    name, K, N = w.linears[layer]
    a, wt = wl.layer_inputs(w, layer)
    say("bf16 prefill gemm qwen3-8b m8192", name, (w.M, N, K))
    y = nv.bf16_gemm(bf16_dev(a), bf16_dev(wt), out_dtype=torch.bfloat16)
    mi, ni = _sample_pairs(w.M, N, 4096, 7 + layer)
    ref = oracle_mod.bf16_gemm_pairs(a, wt, mi, ni)
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy()
    parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"bf16 {name} sampled")


@pytest.mark.parametrize("layer", range(4))
def test_qwen3_32b_m16384_sampled(nv, oracle_mod, layer):
    """Qwen3-32B prefill linears at 16384 tokens (dynamic-alpha activation
    quantizer + NVFP4 GEMM, BF16 output); quantized activation bit-exact in
    full, 4100 sampled outputs against the exact oracle."""
    import torch

    w = wl.WORKLOADS["qwen3_32b_m16384"]
    name, K, N = w.linears[layer]
    a, wt = wl.layer_inputs(w, layer)
    A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
    say("nvfp4 gemm qwen3-32b m16384", name, (w.M, N, K))
    ac, asc, aal = nv.nvfp4_quantize(bf16_dev(a))
    del a
    assert np.array_equal(host(asc), A[1]) and np.array_equal(host(ac), A[0]) and host(aal)[0] == A[2]
    wc, wsc, wal = _dev_operand(W)
    y = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.bfloat16)
    mi, ni = _sample_pairs(w.M, N, 4096, 300 + layer)
    ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].float().cpu().numpy()
    parity.assert_gemm_close(got, ref, parity.GEMM_TOL_BF16, f"32b {name} sampled")


@pytest.mark.parametrize("M", [512, 2048, 32768])
def test_phase_split_prefill_token_counts(nv, oracle_mod, M):
    """NVFP4 prefill at the phase-split token counts (the 8192 case is covered
    above), Qwen3-8B QKV and down projections, against the oracle."""
    import torch

    for layer in (0, 3):
        name, K, N = wl.QWEN3_8B_LINEARS[layer]
        a = wl.activations(M, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 0))
        wt = wl.weights(N, K, wl.rng(wl.PHASE_SPLIT_CONFIG_ID, layer, 1))
        A, W = oracle_mod.quantize(a), oracle_mod.quantize(wt)
        say("phase split prefill", name, (M, N, K))
        ac, asc, aal = nv.nvfp4_quantize(bf16_dev(a))
        assert np.array_equal(host(ac), A[0]) and np.array_equal(host(asc), A[1])
        wc, wsc, wal = _dev_operand(W)
        y = nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out_dtype=torch.float32)
        mi, ni = _sample_pairs(M, N, 2048, M + layer)
        ref = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
        got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
        parity.assert_gemm_close(got, ref, parity.GEMM_TOL_F32, f"phase split {name} M={M}")
