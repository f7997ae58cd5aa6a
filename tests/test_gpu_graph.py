"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): a decode
step (dynamic-alpha quantizer + NVFP4 decode GEMM, and the BF16 decode GEMM)
and a small prefill step are captured once and replayed several times, with
eager work and synchronizations between replays; every replay must reproduce
the eager outputs bit for bit.  The library records only kernel launches (no
memset nodes)."""
import numpy as np
import pytest

from nvfp4_prefill_gemm_amd import workloads as wl
from tests.gpu_util import bf16_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_prefill_gemm_amd import binding

    binding.lib()
    return binding


def test_graph_replays_match_eager(nv):
    import torch

    dev = torch.device("cuda", 0)
    K, N = 4096, 1024
    xd = bf16_dev(wl.activations(8, K, wl.rng(9, 0, 0)))
    xp = bf16_dev(wl.activations(256, K, wl.rng(9, 1, 0)))
    wb = bf16_dev(wl.weights(N, K, wl.rng(9, 0, 1)))
    wc, wsc, wal = nv.nvfp4_quantize(wb)

    def buffers(M):
        return (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                torch.empty(1, dtype=torch.float32, device=dev),
                torch.empty(max(nv.quantize_workspace_size(M, K), 4), dtype=torch.uint8, device=dev))

    bd, bp = buffers(8), buffers(256)
    yd4 = torch.empty((8, N), dtype=torch.bfloat16, device=dev)
    yd16 = torch.empty((8, N), dtype=torch.float32, device=dev)
    yp = torch.empty((256, N), dtype=torch.bfloat16, device=dev)

    def step():
        nv.nvfp4_quantize(xd, bd[0], bd[1], bd[2], workspace=bd[3])
        nv.nvfp4_gemm(bd[0], bd[1], bd[2], wc, wsc, wal, out=yd4)
        nv.bf16_gemm(xd, wb, out=yd16)
        nv.nvfp4_quantize(xp, bp[0], bp[1], bp[2], workspace=bp[3])
        nv.nvfp4_gemm(bp[0], bp[1], bp[2], wc, wsc, wal, out=yp)

    outs = (bd[0], bd[1], bd[2], yd4, yd16, bp[0], bp[1], bp[2], yp)
    say("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.empty((8, N), dtype=torch.bfloat16, device=dev)
    for rep in range(4):
        for o in outs:
            o.zero_()
        nv.bf16_gemm(xd, wb, out=other)  # eager work between replays
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager result"
    # the eager BF16-output call equals the nearest-even rounding of the captured FP32 output
    assert torch.equal(other, ref[4].to(torch.bfloat16))


def test_graph_replays_decode_packed(nv):
    """A decode step on decode-packed weights (BF16 decode at batch 8, NVFP4
    fused decode at batch 1, quantize-first NVFP4 decode at batch 24 with K
    split over workgroups) captured
    once and replayed with eager work between replays: every replay equals
    the eager result bit for bit."""
    import torch

    dev = torch.device("cuda", 0)
    K, N = 4096, 2048
    wb = bf16_dev(wl.weights(N, K, wl.rng(9, 2, 1)))
    bwp = nv.bf16_decode_pack(wb)
    wpk = nv.nvfp4_decode_pack(*nv.nvfp4_quantize(wb))
    x1 = bf16_dev(wl.activations(1, K, wl.rng(9, 2, 0)))
    x8 = bf16_dev(wl.activations(8, K, wl.rng(9, 3, 0)))
    wb3 = bf16_dev(wl.weights(N, 3 * K, wl.rng(9, 3, 1)))
    wpk3 = nv.nvfp4_decode_pack(*nv.nvfp4_quantize(wb3))
    x8k = bf16_dev(wl.activations(24, 3 * K, wl.rng(9, 4, 0)))
    yb = torch.empty((8, N), dtype=torch.bfloat16, device=dev)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
    y24 = torch.empty((24, N), dtype=torch.float32, device=dev)
    a1 = torch.empty(1, dtype=torch.float32, device=dev)
    a24 = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = torch.empty(max(nv.bf16_gemm_workspace_size(8, N, K), 16), dtype=torch.uint8, device=dev)
    ws1 = torch.empty(max(nv.quant_gemm_workspace_size(1, N, K), 16), dtype=torch.uint8, device=dev)
    ws24 = torch.empty(max(nv.quant_gemm_workspace_size(24, N, 3 * K), 16), dtype=torch.uint8, device=dev)

    def step():
        nv.bf16_gemm_packed(x8, bwp, out=yb, workspace=wsb)
        nv.nvfp4_quant_gemm_packed(x1, wpk, a_alpha=a1, out=y1, workspace=ws1)
        nv.nvfp4_quant_gemm_packed(x8k, wpk3, a_alpha=a24, out=y24, workspace=ws24)

    outs = (yb, y1, y24, a1, a24)
    say("graph packed: eager reference")
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph packed: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        nv.bf16_gemm(x8, wb, out=yb)  # eager work between replays
        torch.cuda.synchronize()
        say("graph packed: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager result"
