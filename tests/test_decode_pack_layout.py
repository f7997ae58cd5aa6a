"""CPU checks of the decode-packed weight layout: the reshaped form the GPU
tests compare against equals the element-by-element definition of
include/nvfp4.h, the library's size query agrees with it, and the binding
rejects malformed packed weights before any device call."""
import numpy as np
import pytest

from tests import decode_pack_ref as ref


@pytest.mark.parametrize("N,K", [(1, 128), (16, 256), (20, 384), (47, 512)])
def test_reshaped_layout_equals_definition(N, K):
    g = np.random.default_rng(N * 1000 + K)
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(0, 127, size=(N, K // 16), dtype=np.uint8)
    assert np.array_equal(ref.pack(codes, scales), ref.pack_loops(codes, scales))


def test_layout_places_known_bytes():
    """Hand-checked positions: row 17 (group 1, lane 1 and 17, 33, 49), chunk 1."""
    N, K = 40, 256
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.zeros((N, K // 16), dtype=np.uint8)
    codes[17, 64 + 16 * 2 + 3] = 0xAB   # chunk 1, quarter 2, byte 3 -> lane 16 * 2 + 1 = 33
    scales[17, 8 + 5] = 0x4C            # chunk 1, scale 5 of row r = 1
    p = ref.pack(codes, scales)
    base = (1 * 2 + 1) * ref.BLOCK      # group 1, chunk 1 of 2
    assert p[base + 16 * 33 + 3] == 0xAB and p[base + 1024 + 8 * 1 + 5] == 0x4C
    assert np.count_nonzero(p) == 2
    assert p.size == 3 * 2 * ref.BLOCK


@pytest.mark.parametrize("N,K", [(1, 32), (16, 64), (21, 96), (40, 256)])
def test_bf16_reshaped_layout_equals_definition(N, K):
    g = np.random.default_rng(N * 100 + K)
    w = g.integers(0, 65536, size=(N, K), dtype=np.uint16)
    assert np.array_equal(ref.pack_bf16(w), ref.pack_bf16_loops(w))


def test_bf16_layout_places_known_bytes():
    """Row 18 (group 1, r = 2), element 45 (step 1, quarter 1, element 5):
    lane 16 + 2, bytes 10 and 11 of its 16."""
    N, K = 20, 64
    w = np.zeros((N, K), dtype=np.uint16)
    w[18, 45] = 0xBEEF
    p = ref.pack_bf16(w)
    base = (1 * 2 + 1) * ref.BF16_BLOCK
    assert p[base + 16 * 18 + 10] == 0xEF and p[base + 16 * 18 + 11] == 0xBE
    assert np.count_nonzero(p) == 2 and p.size == 2 * 2 * ref.BF16_BLOCK


@pytest.fixture(scope="module")
def nvb():
    from nvfp4_prefill_gemm_amd import binding

    import os
    if not os.path.exists(binding.LIB_PATH):
        from nvfp4_prefill_gemm_amd import build

        build.build()
    binding.lib()
    return binding


def test_pack_size_matches_layout(nvb):
    for N, K in ((1, 128), (40, 256), (1000, 4096), (24576, 4096), (4096, 12288)):
        assert nvb.decode_pack_size(N, K) == ((N + 15) // 16) * (K // 128) * ref.BLOCK
    assert nvb.decode_pack_size(0, 128) == 0 and nvb.decode_pack_size(16, 96) == 0


def test_bf16_pack_size_matches_layout(nvb):
    for N, K in ((1, 32), (40, 256), (24576, 4096), (4096, 12288)):
        assert nvb.bf16_decode_pack_size(N, K) == ((N + 15) // 16) * (K // 32) * ref.BF16_BLOCK
    assert nvb.bf16_decode_pack_size(16, 40) == 0


def test_binding_rejects_malformed_packed_weights(nvb):
    import torch

    codes = torch.zeros((40, 128), dtype=torch.uint8)
    scales = torch.zeros((40, 16), dtype=torch.uint8)
    alpha = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError):  # K = 256 is fine, but host tensors
        nvb.nvfp4_decode_pack(codes, scales, alpha)
    with pytest.raises(ValueError):  # K = 96 is not a multiple of 128
        nvb.nvfp4_decode_pack(torch.zeros((40, 48), dtype=torch.uint8), torch.zeros((40, 6), dtype=torch.uint8),
                              alpha)
    good = nvb.DecodePackedWeight(torch.zeros(nvb.decode_pack_size(40, 256), dtype=torch.uint8), alpha, 40, 256)
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        nvb.nvfp4_quant_gemm_packed(x, (good.packed, alpha, 40, 256))
    with pytest.raises(ValueError):  # wrong byte count
        nvb.nvfp4_quant_gemm_packed(x, good._replace(packed=good.packed[:-16]))
    with pytest.raises(ValueError):  # K disagrees
        nvb.nvfp4_quant_gemm_packed(torch.zeros((2, 384), dtype=torch.bfloat16), good)
    with pytest.raises(ValueError):  # host tensors
        nvb.nvfp4_quant_gemm_packed(x, good)
    bwp = nvb.Bf16PackedWeight(torch.zeros(nvb.bf16_decode_pack_size(40, 256), dtype=torch.uint8), 40, 256)
    with pytest.raises(TypeError):
        nvb.bf16_gemm_packed(x, good)
    with pytest.raises(ValueError):  # K disagrees
        nvb.bf16_gemm_packed(torch.zeros((2, 288), dtype=torch.bfloat16), bwp)
    with pytest.raises(ValueError):  # K % 32
        nvb.bf16_decode_pack(torch.zeros((4, 40), dtype=torch.bfloat16))
    with pytest.raises(ValueError):  # host tensors
        nvb.bf16_gemm_packed(x, bwp)
