"""Pins for the oracle's MXFP4 functions (CPU only).

MXFP4 = E2M1 elements with one E8M0 (power-of-two) scale per 32 elements, the
coarser microscaling format Mix-Quant Section 3.3 contrasts with NVFP4.  The
rounding rule is the OCP MX v1.0 conversion (shared exponent =
floor(log2(amax)) - 2, clamped to [-127, 127]; nearest-even E2M1 with
saturation).  Pins: E8M0 landmarks from the format definition, hand-derived
blocks for the shared-exponent rule and saturation, constructed round trips,
exact rational brute force for the GEMM, and a float64 matmul cross-check.
"""
from fractions import Fraction

import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _val(c):
    c = int(c)
    return -E2M1[c & 7] if c & 8 else E2M1[c & 7]


def _bits(x):
    x = np.asarray(x, dtype=np.float32)
    b = wl.to_bf16_bits(x)
    assert np.array_equal(wl.bf16_bits_to_f32(b), x)
    return b


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def test_e8m0_landmarks(oracle_mod):
    # OCP MX v1.0 E8M0: unsigned exponent, bias 127, 0xFF = NaN
    assert oracle_mod.e8m0_value(0x7F) == 1.0
    assert oracle_mod.e8m0_value(0x80) == 2.0
    assert oracle_mod.e8m0_value(0x00) == 2.0 ** -127
    assert oracle_mod.e8m0_value(0xFE) == 2.0 ** 127
    assert np.isnan(oracle_mod.e8m0_value(0xFF))


@pytest.mark.parametrize("amax,scale_code,amax_code", [
    (1.0, 127 - 2, 0x6),     # floor(log2 1) = 0 -> 2^-2; 1 / 0.25 = 4
    (1.5, 127 - 2, 0x7),     # 1.5 / 0.25 = 6
    (1.75, 127 - 2, 0x7),    # 7 saturates to 6
    (1.9375, 127 - 2, 0x7),  # 7.75 saturates to 6
    (2.0, 127 - 1, 0x6),     # next binade
    (3.0, 127 - 1, 0x7),
    (2.0 ** -20, 127 - 22, 0x6),
    (2.0 ** -130, 0, 0x0),   # shared exponent -132 clamps to -127: 2^-130 / 2^-127 = 0.125 -> 0
])
def test_shared_exponent_rule(oracle_mod, amax, scale_code, amax_code):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 5] = amax
    x[0, 6] = -amax / 2
    codes, scales = oracle_mod.mx_quantize(_bits(x))
    assert scales[0, 0] == scale_code
    u = _unpack(codes)[0]
    assert u[5] == amax_code
    assert u[0] == 0 and u[31] == 0


def test_zero_block_and_signed_zero(oracle_mod):
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, 3] = -0.0
    x[1, 40] = 1.0
    codes, scales = oracle_mod.mx_quantize(_bits(x))
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    u = _unpack(codes)
    assert u[0, 3] == 0x8 and u[0].sum() == 0x8


def test_ties_round_to_even(oracle_mod):
    # amax 4 -> shared exponent 0 -> elements are used as is
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 4.0
    x[0, 1:8] = ties
    x[0, 8:15] = -np.array(ties, dtype=np.float32)
    codes, scales = oracle_mod.mx_quantize(_bits(x))
    assert scales[0, 0] == 127
    u = _unpack(codes)[0]
    assert list(u[1:8]) == [0, 2, 2, 4, 4, 6, 6]
    assert list(u[8:15]) == [8 | c for c in [0, 2, 2, 4, 4, 6, 6]]


@pytest.mark.parametrize("seed", [0, 1])
def test_roundtrip_constructed(oracle_mod, seed):
    """x = 2^s * q with max |q| in {4, 6} per block reproduces s and q exactly."""
    g = np.random.default_rng(seed)
    rows, nb = 8, 6
    s = g.integers(-40, 40, size=(rows, nb))
    q = g.integers(0, 16, size=(rows, nb * 32)).astype(np.uint8)
    q[q == 8] = 0
    top = g.choice([0x6, 0x7], size=(rows, nb))  # 4 or 6
    for r in range(rows):
        for b in range(nb):
            blk = q[r, b * 32:(b + 1) * 32]
            blk[np.abs(np.vectorize(_val)(blk)) > E2M1[top[r, b]]] = top[r, b]
            blk[g.integers(0, 32)] = top[r, b] | (8 * g.integers(0, 2))
    vals = np.vectorize(_val, otypes=[np.float64])(q) * np.repeat(2.0 ** s, 32, axis=1)
    xb = _bits(vals.astype(np.float32))
    codes, scales = oracle_mod.mx_quantize(xb)
    assert np.array_equal(scales.astype(int) - 127, s)
    assert np.array_equal(_unpack(codes), q)
    assert np.array_equal(oracle_mod.mx_dequantize(codes, scales), vals)


@pytest.mark.parametrize("K", [32, 64, 96])
def test_mx_gemm_bruteforce_rational(oracle_mod, K):
    g = np.random.default_rng(K)
    M, N = 3, 4
    qa = g.integers(0, 16, size=(M, K))
    qw = g.integers(0, 16, size=(N, K))
    sa = g.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
    sw = g.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    pack = lambda q: (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    y = oracle_mod.mx_gemm(pack(qa), sa, pack(qw), sw)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(2) ** (int(sa[m, k // 32]) - 127) * Fraction(_val(qa[m, k]))
                        * Fraction(2) ** (int(sw[n, k // 32]) - 127) * Fraction(_val(qw[n, k])))
            assert abs(y[m, n] - float(acc)) <= 2.0 ** -50 * abs(float(acc)) + 1e-300


def test_mx_gemm_matches_dequantized_matmul(oracle_mod):
    g = np.random.default_rng(3)
    a = wl.to_bf16_bits(g.standard_normal((40, 256), dtype=np.float32))
    w = wl.to_bf16_bits(g.standard_normal((24, 256), dtype=np.float32) * 0.02)
    A, W = oracle_mod.mx_quantize(a), oracle_mod.mx_quantize(w)
    y = oracle_mod.mx_gemm(*A, *W)
    ref = oracle_mod.mx_dequantize(*A) @ oracle_mod.mx_dequantize(*W).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)
    mi, ni = np.array([0, 39, 7]), np.array([23, 0, 11])
    assert np.array_equal(oracle_mod.mx_gemm_pairs(*A, *W, mi, ni), y[mi, ni])
