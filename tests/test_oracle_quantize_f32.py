"""Pins for the oracle's FP32-input quantizer: Eq. 3 and Eq. 2 (Mix-Quant
Section 3.3) applied to an FP32 tensor such as a GEMM output, each value
taken at full FP32 precision.

Anchors: hand-derived codes for values a few FP32 ulps either side of E2M1
and E4M3 rounding ties (values BF16 cannot hold, so an implementation that
rounded to BF16 first fails), exact ties to even, constructed tensors that
must round-trip, and equality with the BF16 quantizer wherever the input is
BF16-representable.
"""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def _block(values):
    v = np.zeros(16, dtype=np.float32)
    v[: len(values)] = values
    return v


def test_e2m1_ties_and_neighbours_at_fp32_precision(oracle_mod):
    """alpha = 1 and a block amax of 6 give sigma = 1 (code 0x38) and divisor
    1, so each value's code is its own E2M1 rounding: ties (0.25, 0.75, 1.25,
    2.5, 3.5, 5) go to the even mantissa; a few 2^-20 either side decides."""
    e = np.float32(2.0 ** -20)
    vals = [6.0, 0.75, 0.75 + e, 0.75 - e, 1.25, 1.25 + e, 2.5, 2.5 - 2 * e, 3.5, 3.5 + 4 * e, 5.0,
            5.0 + 4 * e, -0.25, -0.25 - e, 5.75, -6.0]
    want = [0x7, 0x2, 0x2, 0x1, 0x2, 0x3, 0x4, 0x4, 0x6, 0x6, 0x6, 0x7, 0x8, 0x9, 0x7, 0xF]
    x = _block([np.float32(v) for v in vals])[None, :]
    x[0, 0] = 6.0
    codes, scales, _ = oracle_mod.quantize_f32(x, alpha=1.0)
    assert scales[0, 0] == 0x38
    got = _unpack(codes)[0]
    assert got.tolist() == want


def test_e4m3_scale_tie_at_fp32_precision(oracle_mod):
    """amax = 6 * 1.0625 is the E4M3 tie between 1.0 and 1.125 (to even:
    1.0, code 0x38); 6 * (1.0625 + 2^-20) rounds up to 1.125 (code 0x39)."""
    a = np.float32(6.0 * 1.0625)
    b = np.float32(6.0) * np.float32(1.0625 + 2.0 ** -20)
    assert b > a
    x = np.stack([_block([a, 1.0]), _block([b, 1.0])])
    _, scales, _ = oracle_mod.quantize_f32(x, alpha=1.0)
    assert scales[:, 0].tolist() == [0x38, 0x39]


def test_dynamic_alpha_over_fp32_values(oracle_mod):
    """Dynamic alpha is amax / 2688 over the FP32 values themselves."""
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 17] = -2688.0 * np.float32(1.0 + 2.0 ** -20)
    _, _, alpha = oracle_mod.quantize_f32(x)
    assert alpha == np.float32(np.float32(2688.0 * np.float32(1.0 + 2.0 ** -20)) / np.float32(2688.0))
    x[1, 17] = -2688.0 / 8
    assert oracle_mod.quantize_f32(x)[2] == np.float32(0.125)


@pytest.mark.parametrize("log2_alpha", [-12, 0, 5])
def test_roundtrip_constructed(oracle_mod, log2_alpha):
    """x = alpha * sigma_b * q with alpha = 2^j (static), max |q| = 6 per
    block: codes and scales are reproduced exactly."""
    g = np.random.default_rng(40 + log2_alpha)
    rows, cols = 12, 128
    e4m3 = oracle_mod.e4m3_table()
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    sc = g.integers(1, 127, size=(rows, cols // 16))
    q = g.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    q[q == 0x8] = 0
    q[:, ::16] = 0x7
    x = (2.0 ** log2_alpha) * np.repeat(e4m3[sc], 16, axis=1) * e2m1[q]
    codes, scales, _ = oracle_mod.quantize_f32(x.astype(np.float32), alpha=float(2.0 ** log2_alpha))
    assert np.array_equal(scales, sc.astype(np.uint8))
    assert np.array_equal(_unpack(codes), q)


@pytest.mark.parametrize("alpha", [None, 0.013])
def test_matches_bf16_quantizer_on_bf16_values(oracle_mod, alpha):
    """On BF16-representable inputs both entry points quantize the same values."""
    g = np.random.default_rng(3)
    xb = wl.to_bf16_bits(g.standard_t(3.0, size=(40, 96)).astype(np.float32))
    xf = wl.bf16_bits_to_f32(xb)
    a = oracle_mod.quantize(xb, alpha=alpha)
    b = oracle_mod.quantize_f32(xf, alpha=alpha)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]
