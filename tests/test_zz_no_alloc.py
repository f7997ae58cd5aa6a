"""GPU: nvfp4_quantize_noalloc, the entry point that allocates nothing (its
amax partials live in the library's per-GPU scratch array), against
nvfp4_quantize with a caller workspace: codes, scales and the tensor scale
bit for bit, on two calls in a row, the second on a smaller tensor (the
scratch keeps the first call's partials, which the second must not see).
"""
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


def _outputs(rows, cols):
    import torch

    return (torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
            torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"))


def _same(got, ref, what):
    for g, r, name in zip(got, ref, ("codes", "scales", "alpha")):
        assert np.array_equal(host(g), host(r)), f"{what}: {name} differ"


@pytest.mark.parametrize("static", [False, True])
def test_noalloc_matches_workspace_entry_point(nv, static):
    rng = np.random.default_rng(2024)
    # first call: a large activation (many amax partials, large values);
    # second: a smaller one with much smaller values, so stale partials from
    # the first call would change its tensor scale
    shapes = ((4096, 12288, 8.0), (300, 4112, 0.01))
    for rows, cols, scale in shapes:
        x = bf16_dev(wl.to_bf16_bits(rng.standard_normal((rows, cols), dtype=np.float32) * scale))
        ref = nv.nvfp4_quantize(x, *_outputs(rows, cols)[:2],
                                alpha=f32_dev([0.37 * scale]) if static else None, static_alpha=static)
        out = _outputs(rows, cols)
        if static:
            out[2].copy_(ref[2])
        say("quantize_noalloc", rows, cols, "static" if static else "dynamic")
        got = nv.nvfp4_quantize_noalloc(x, *out, static_alpha=static)
        _same(got, ref, f"noalloc {rows}x{cols}")
        if not static:
            assert float(host(got[2])[0]) == np.float32(float(host(x.abs().max().float().reshape(1))[0]) / 2688.0)


def test_noalloc_strided_rows_and_empty(nv):
    import torch

    rng = np.random.default_rng(7)
    big = bf16_dev(wl.to_bf16_bits(rng.standard_normal((64, 1040), dtype=np.float32)))
    x = big[:, :1024]
    ref = nv.nvfp4_quantize(x)
    say("quantize_noalloc strided")
    got = nv.nvfp4_quantize_noalloc(x, *_outputs(64, 1024))
    _same(got, ref, "noalloc strided")
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    nv.nvfp4_quantize_noalloc(e, *_outputs(0, 64))
