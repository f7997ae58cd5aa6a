"""GPU: every GEMM entry point writes into a row-strided output (ld_out > N)
exactly what it writes into a contiguous one, and leaves the padding columns
alone.  Decode (M = 5) and tile (M = 300) kernels, FP32 and BF16 output."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests.gpu_util import bf16_dev, say

pytestmark = pytest.mark.gpu

PAD = 40
SENTINEL = 12345.0


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def _check(fn, M, N, what):
    import torch

    for dt in (torch.float32, torch.bfloat16):
        say("strided output", what, dt)
        ref = fn(None, dt)
        big = torch.full((M, N + PAD), SENTINEL, dtype=dt, device="cuda")
        view = big[:, :N]
        assert view.stride(0) == N + PAD
        fn(view, dt)
        assert torch.equal(view, ref), f"{what} ({dt}): strided output differs"
        pad = torch.full((M, PAD), SENTINEL, dtype=dt, device="cuda")
        assert torch.equal(big[:, N:], pad), f"{what} ({dt}): padding columns written"


@pytest.mark.parametrize("M", [5, 300])
def test_gemms_strided_out(nv, M):
    N, K = 520, 512
    g = np.random.default_rng(M + 11)
    x = bf16_dev(wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32)))
    w = bf16_dev(wl.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * 0.02))
    ac, asc, aal = nv.nvfp4_quantize(x)
    wc, wsc, wal = nv.nvfp4_quantize(w)
    _check(lambda out, dt: nv.nvfp4_gemm(ac, asc, aal, wc, wsc, wal, out=out, out_dtype=dt), M, N,
           f"nvfp4_gemm M={M}")
    _check(lambda out, dt: nv.nvfp4_quant_gemm(x, wc, wsc, wal, out=out, out_dtype=dt)[0], M, N,
           f"nvfp4_quant_gemm M={M}")
    _check(lambda out, dt: nv.bf16_gemm(x, w, out=out, out_dtype=dt), M, N, f"bf16_gemm M={M}")
    mac, masc = nv.mxfp4_quantize(x)[:2]
    mwc, mwsc = nv.mxfp4_quantize(w)[:2]
    _check(lambda out, dt: nv.mxfp4_gemm(mac, masc, mwc, mwsc, out=out, out_dtype=dt), M, N, f"mxfp4_gemm M={M}")
