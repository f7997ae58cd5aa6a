"""GPU parity of the NVFP4 quantizer against the oracle: codes, scales and the
tensor scale must match bit for bit (Mix-Quant Section 3.3, Eq. 2 and Eq. 3)."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests.gpu_util import bf16_dev, f32_dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _gpu_quant(nv, xb, alpha=None, ld=None):
    import torch

    x = bf16_dev(xb)
    if ld is not None and ld != xb.shape[1]:
        big = torch.zeros((xb.shape[0], ld), dtype=torch.bfloat16, device="cuda")
        big[:, : xb.shape[1]] = x
        x = big[:, : xb.shape[1]]
    if alpha is None:
        c, s, a = nv.nvfp4_quantize(x)
    else:
        c, s, a = nv.nvfp4_quantize(x, alpha=f32_dev([alpha]), static_alpha=True)
    return host(c), host(s), np.float32(host(a)[0])


def _assert_same(got, want, what):
    c, s, a = got
    wc, ws, wa = want
    assert a.view(np.uint32) == np.float32(wa).view(np.uint32), f"{what}: alpha {a!r} != {wa!r}"
    bad = np.argwhere(s != ws)
    assert bad.size == 0, f"{what}: {len(bad)} scale mismatches, first {bad[:3].tolist()}"
    bad = np.argwhere(c != wc)
    assert bad.size == 0, f"{what}: {len(bad)} code-byte mismatches, first {bad[:3].tolist()}"


def test_tiny_config_bit_exact(nv, oracle_mod):
    w = wl.WORKLOADS["tiny"]
    a, wt = wl.layer_inputs(w, 0)
    for name, xb in (("A", a), ("W", wt)):
        say("quantize tiny", name, xb.shape)
        _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), f"tiny {name}")


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (5, 1040), (130, 272), (257, 4096)])
def test_ragged_shapes(nv, oracle_mod, rows, cols):
    g = np.random.default_rng(rows * 1000 + cols)
    xb = wl.to_bf16_bits(g.standard_normal((rows, cols), dtype=np.float32) * 2)
    say("quantize ragged", rows, cols)
    _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), f"{rows}x{cols}")


def test_static_alpha_and_strided_rows(nv, oracle_mod):
    g = np.random.default_rng(5)
    xb = wl.to_bf16_bits(g.standard_t(4.0, size=(64, 512)).astype(np.float32))
    for alpha in (0.0123, 1.0, 3.0e-6):
        say("quantize static alpha", alpha)
        _assert_same(_gpu_quant(nv, xb, alpha=alpha), oracle_mod.quantize(xb, alpha=alpha), f"static {alpha}")
    say("quantize strided ld=520")
    _assert_same(_gpu_quant(nv, xb, ld=520), oracle_mod.quantize(xb), "strided")


def test_static_alpha_extreme_quotients(nv, oracle_mod):
    """Static tensor scales far below the data: block scales saturate at 448
    and x / (alpha * sigma) exceeds 2^120 or overflows FP32 (codes clip to
    +-6), next to ordinary blocks; and scales far above it (quotients that
    underflow)."""
    g = np.random.default_rng(21)
    x = g.standard_normal((8, 256)).astype(np.float32)
    x[0] *= np.float32(2.0 ** 120)
    x[1] *= np.float32(2.0 ** 60)
    x[2, :16] = np.float32(-3.0e38)
    x[3] *= np.float32(2.0 ** -100)
    xb = wl.to_bf16_bits(x)
    for alpha in (2.0 ** -105, 2.0 ** -60, 1.0e-30, 2.0 ** 100):
        say("quantize extreme static alpha", alpha)
        _assert_same(_gpu_quant(nv, xb, alpha=alpha), oracle_mod.quantize(xb, alpha=alpha), f"extreme static {alpha}")


def _special_tensor():
    """Zero blocks, signed zeros, E2M1 ties, tiny and saturating blocks (alpha = 1)."""
    rows = []
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    r = np.zeros(64, dtype=np.float32)
    r[0] = 6.0
    r[1:8] = ties
    r[8:15] = -np.array(ties)
    r[15] = -0.0
    r[16:32] = 0.0
    r[20] = -0.0
    r[32:48] = 2.0 ** -100
    r[48] = 6144.0
    r[49] = -6144.0
    rows.append(r)
    for amax_b in (6 * 2.0 ** -11, 6 * 2.0 ** -10, 18 * 2.0 ** -11, 6.375, 2640.0, 6144.0):
        q = np.zeros(64, dtype=np.float32)
        q[3] = amax_b
        q[17] = -amax_b / 3
        q[40] = amax_b * 0.75
        rows.append(q)
    return wl.to_bf16_bits(np.stack(rows))


def test_special_values(nv, oracle_mod):
    xb = _special_tensor()
    say("quantize special values, static alpha 1")
    _assert_same(_gpu_quant(nv, xb, alpha=1.0), oracle_mod.quantize(xb, alpha=1.0), "special static")
    say("quantize special values, dynamic")
    _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), "special dynamic")
    z = np.zeros((8, 32), dtype=np.uint16)
    z[3, 5] = 0x8000  # -0.0
    say("quantize all-zero tensor")
    _assert_same(_gpu_quant(nv, z), oracle_mod.quantize(z), "all zero")


def test_dense_tie_neighbourhood(nv, oracle_mod):
    """Every BF16 value around each E2M1 tie (times a few scales): the quotient
    x / (alpha sigma) lands on and next to the tie points."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    base = wl.to_bf16_bits(ties).astype(np.int32)
    vals = (base[:, None] + np.arange(-6, 7)[None, :]).ravel().astype(np.uint16)
    rows = []
    for scale_exp in (0, -3, 5):
        v = wl.bf16_bits_to_f32(vals) * np.float32(2.0 ** scale_exp)
        v = np.concatenate([v, -v])
        pad = (-len(v)) % 15
        v = np.concatenate([v, np.zeros(pad, dtype=np.float32)]).reshape(-1, 15)
        blk = np.concatenate([np.full((v.shape[0], 1), 6.0 * 2.0 ** scale_exp, dtype=np.float32), v], axis=1)
        rows.append(blk.reshape(-1))
    n = max(len(r) for r in rows)
    x = np.zeros((len(rows), n), dtype=np.float32)
    for i, r in enumerate(rows):
        x[i, : len(r)] = r
    xb = wl.to_bf16_bits(x)
    say("quantize tie neighbourhood", xb.shape)
    _assert_same(_gpu_quant(nv, xb, alpha=1.0), oracle_mod.quantize(xb, alpha=1.0), "ties static")
    _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), "ties dynamic")


def test_e4m3_scale_grid(nv, oracle_mod):
    """Eq. 3 on every BF16 block amax from 2^-14 to 1024: with the static
    tensor scale fl32(1/6), t = fl32(alpha * 6) is exactly 1, so s equals the
    block amax and the E4M3 projection meets every tie and neighbour of the
    normal and subnormal grids and the saturation at 448; the dynamic run
    (tensor amax 1024) gives a non-power-of-two t."""
    alpha = np.float32(1.0) / np.float32(6.0)
    assert np.float32(alpha * np.float32(6.0)) == np.float32(1.0)
    lo, hi = (int(b) for b in wl.to_bf16_bits(np.array([2.0 ** -14, 1024.0], dtype=np.float32)))
    amax = wl.bf16_bits_to_f32(np.arange(lo, hi + 1, dtype=np.uint32).astype(np.uint16))
    nb = -(-len(amax) // 16) * 16
    amax = np.concatenate([amax, np.full(nb - len(amax), 1.0, dtype=np.float32)])
    frac = np.array([1, -0.5, 1 / 3, -0.75, 0.25, 0, -0.125, 0.9, -0.6, 0.1, 0.05, -0.3, 0.7, -0.95, 0.2, 0.4],
                    dtype=np.float32)
    x = (amax[:, None] * frac[None, :]).reshape(nb // 16, 256)
    xb = wl.to_bf16_bits(x)
    say("quantize E4M3 scale grid", xb.shape)
    _assert_same(_gpu_quant(nv, xb, alpha=float(alpha)), oracle_mod.quantize(xb, alpha=float(alpha)), "grid static")
    _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), "grid dynamic")


@pytest.mark.parametrize("layer", range(4))
def test_qwen3_8b_m8192_full_tensors(nv, oracle_mod, layer):
    w = wl.WORKLOADS["qwen3_8b_m8192"]
    a, wt = wl.layer_inputs(w, layer)
    for name, xb in (("A", a), ("W", wt)):
        say("quantize qwen3-8b m8192", w.linears[layer][0], name, xb.shape)
        _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), f"layer {layer} {name}")


def test_student_t_long_prefill_full_tensor(nv, oracle_mod):
    w = wl.WORKLOADS["qwen3_8b_m32768_t4"]
    _, K, _ = w.linears[3]
    xb = wl.activations(w.M, K, wl.rng(w.config_id, 3, 0), w.act_dist)
    say("quantize student-t m32768 down-proj input", xb.shape)
    _assert_same(_gpu_quant(nv, xb), oracle_mod.quantize(xb), "student-t 32768x12288")


@pytest.mark.parametrize("rows,cols,ld_pad", [(8, 12288, 0), (32, 4096, 0), (33, 4096, 0), (17, 4112, 24),
                                              (3, 40960, 8), (4, 8192, 0), (16, 4096, 0), (16, 4096, 8),
                                              (15, 4368, 0), (3, 21856, 24), (64, 4096, 0)])
def test_decode_batch_sizes_amax_placement(nv, oracle_mod, rows, cols, ld_pad):
    """Decode-batch-sized tensors on both sides of the single-launch limit
    (at most 65536 elements: every workgroup reads the whole tensor in up to
    two rounds of loads; above it the amax pass + quantize pass, few
    workgroups), strided rows: the largest magnitude placed in the last row's
    tail, then in the first row, so every round and every workgroup's partial
    maximum must count."""
    g = np.random.default_rng(rows * 7 + cols)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    for where in ((rows - 1, cols - 3), (0, 1)):
        xx = x.copy()
        xx[where] = 97.0
        xb = wl.to_bf16_bits(xx)
        say("quantize decode-batch sizes", rows, cols, ld_pad, where)
        _assert_same(_gpu_quant(nv, xb, ld=cols + ld_pad), oracle_mod.quantize(xb), f"{rows}x{cols} max at {where}")
