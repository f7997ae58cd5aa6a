"""Pins for the oracle's GEMMs (CPU only).

The product of two NVFP4 tensors is Y = xhatA @ xhatW^T with xhat from Eq. 2 of
Mix-Quant Section 3.3.  Pins: a case that reduces to a plain float64 matmul
(all scales 1), brute force in exact rational arithmetic on tiny shapes, the
textbook FP32 summation error bound for the literal FP32 form, and numpy's
float64 matmul for the BF16 decode GEMM.  A planted-mistake test shows the
gate catches a wrong scale index and a transposed operand.
"""
from fractions import Fraction

import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests import parity

E2M1_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pack(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _val(c):
    c = int(c)
    v = E2M1_POS[c & 7]
    return -v if c & 8 else v


def test_unit_scales_reduce_to_float64_matmul(oracle_mod):
    g = np.random.default_rng(1)
    M, N, K = 9, 7, 64
    qa = g.integers(0, 16, size=(M, K))
    qw = g.integers(0, 16, size=(N, K))
    one = np.full((M, K // 16), 0x38, dtype=np.uint8)
    onew = np.full((N, K // 16), 0x38, dtype=np.uint8)
    y = oracle_mod.gemm_exact(_pack(qa), one, 1.0, _pack(qw), onew, 1.0)
    va = np.vectorize(_val, otypes=[np.float64])(qa).astype(np.float64)
    vw = np.vectorize(_val, otypes=[np.float64])(qw).astype(np.float64)
    assert np.array_equal(y, va @ vw.T)  # all partial sums are exact in float64


@pytest.mark.parametrize("K", [16, 32, 64])
def test_bruteforce_rational(oracle_mod, K):
    g = np.random.default_rng(K)
    M, N = 4, 3
    qa = g.integers(0, 16, size=(M, K))
    qw = g.integers(0, 16, size=(N, K))
    qa[0, :] = 7   # edge codes: all +6
    qw[0, :] = 15  # all -6
    sa = g.integers(0, 127, size=(M, K // 16)).astype(np.uint8)
    sw = g.integers(0, 127, size=(N, K // 16)).astype(np.uint8)
    sa[0, 0], sw[0, 0], sa[1, 0] = 0x7E, 0x7E, 0x01  # 448, 448, 2^-9
    alpha_a, alpha_w = np.float32(0.013), np.float32(3.5e-5)
    e4 = oracle_mod.e4m3_table()
    y = oracle_mod.gemm_exact(_pack(qa), sa, alpha_a, _pack(qw), sw, alpha_w)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                xa = Fraction(float(alpha_a)) * Fraction(e4[sa[m, k // 16]]) * Fraction(_val(qa[m, k]))
                xw = Fraction(float(alpha_w)) * Fraction(e4[sw[n, k // 16]]) * Fraction(_val(qw[n, k]))
                acc += xa * xw
            ref = float(acc)
            assert abs(y[m, n] - ref) <= 4 * 2.0 ** -53 * abs(ref), (m, n, y[m, n], ref)


def _tiny_operands(oracle_mod):
    w = wl.WORKLOADS["tiny"]
    a, wt = wl.layer_inputs(w, 0)
    A = oracle_mod.quantize(a)
    W = oracle_mod.quantize(wt)
    return A, W


def test_exact_matches_dequantized_float64_matmul(oracle_mod):
    A, W = _tiny_operands(oracle_mod)
    y = oracle_mod.gemm_exact(*A, *W)
    xa = oracle_mod.dequantize(*A)
    xw = oracle_mod.dequantize(*W)
    ref = xa @ xw.T
    bound = 256 * 2.0 ** -52 * (np.abs(xa) @ np.abs(xw).T)
    assert np.all(np.abs(y - ref) <= bound)


def test_fp32_literal_within_summation_bound(oracle_mod):
    A, W = _tiny_operands(oracle_mod)
    K = A[0].shape[1] * 2
    y = oracle_mod.gemm_exact(*A, *W)
    y32 = oracle_mod.gemm_fp32(*A, *W)
    xa = oracle_mod.dequantize(*A)
    xw = oracle_mod.dequantize(*W)
    # x_hat rounded to FP32 (1 ulp each), FP32 products and K sequential FP32 adds
    gamma = (K + 3) * 2.0 ** -24 / (1 - (K + 3) * 2.0 ** -24)
    bound = gamma * (np.abs(xa) @ np.abs(xw).T)
    assert np.all(np.abs(y32.astype(np.float64) - y) <= bound)
    parity.assert_gemm_close(y32, y, parity.GEMM_TOL_F32, "fp32 literal vs exact")


def test_exact_pairs_match_full(oracle_mod):
    A, W = _tiny_operands(oracle_mod)
    y = oracle_mod.gemm_exact(*A, *W)
    g = np.random.default_rng(5)
    mi = g.integers(0, y.shape[0], 50)
    ni = g.integers(0, y.shape[1], 50)
    yp = oracle_mod.gemm_exact_pairs(*A, *W, mi, ni)
    assert np.array_equal(yp, y[mi, ni])


def test_bf16_gemm_matches_numpy(oracle_mod):
    g = np.random.default_rng(9)
    a = wl.to_bf16_bits(g.standard_normal((17, 96), dtype=np.float32))
    w = wl.to_bf16_bits(g.standard_normal((23, 96), dtype=np.float32) * 0.02)
    y = oracle_mod.bf16_gemm(a, w)
    ref = wl.bf16_bits_to_f32(a).astype(np.float64) @ wl.bf16_bits_to_f32(w).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-15)
    mi, ni = np.array([0, 16, 3]), np.array([22, 0, 5])
    assert np.array_equal(oracle_mod.bf16_gemm_pairs(a, w, mi, ni), y[mi, ni])


def test_gate_catches_planted_mistakes(oracle_mod):
    """Mistakes planted in oracle outputs on the CPU must fail the GEMM gate."""
    A, W = _tiny_operands(oracle_mod)
    y = oracle_mod.gemm_exact(*A, *W)
    # (1) scales of one operand shifted by one block
    bad_scales = np.roll(W[1], 1, axis=1)
    y1 = oracle_mod.gemm_exact(*A, W[0], bad_scales, W[2])
    assert parity.floored_rel_err(y1, y) > 1e-2
    # (2) nibble order swapped in A
    swapped = ((A[0] >> 4) | (A[0] << 4)).astype(np.uint8)
    y2 = oracle_mod.gemm_exact(swapped, A[1], A[2], *W)
    assert parity.floored_rel_err(y2, y) > 1e-2
    # (3) a single flipped output sign
    y3 = y.copy()
    y3[5, 7] = -y3[5, 7]
    assert parity.floored_rel_err(y3, y) > 1e-3
    # (4) a missing tensor scale
    y4 = oracle_mod.gemm_exact(*A, W[0], W[1], 1.0)
    assert parity.floored_rel_err(y4, y) > 1e-2
