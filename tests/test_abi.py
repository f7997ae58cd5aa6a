"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nvfp4.h declares, and rejects bad arguments with the
documented status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from nvfp4_prefill_gemm_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from nvfp4_prefill_gemm_amd import build

        build.build()
    return binding.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_quant_gemm", "bf16_gemm", "nvfp4_last_error",
              "nvfp4_abi_version", "nvfp4_quantize_workspace_size", "nvfp4_quant_gemm_workspace_size",
              "nvfp4_gemm_workspace_size", "bf16_gemm_workspace_size", "nvfp4_quantize_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_abi_version(L):
    assert L.nvfp4_abi_version() == 3


def test_workspace_sizes(L):
    assert L.nvfp4_quantize_workspace_size(0, 4096) == 0
    assert L.nvfp4_quantize_workspace_size(8192, 4096) > 0
    assert L.nvfp4_quantize_workspace_size(8192, 4096) <= 4096
    # quantize into the workspace, then the GEMM: codes + scales + amax partials (256-byte aligned parts)
    q = L.nvfp4_quant_gemm_workspace_size(128, 512, 256)
    assert q >= 128 * 256 // 2 + 128 * 256 // 16 + L.nvfp4_quantize_workspace_size(128, 256)
    # decode batches: at least the dynamic alpha's partials
    assert L.nvfp4_quant_gemm_workspace_size(8, 4096, 4096) >= L.nvfp4_quantize_workspace_size(8, 4096)
    # tile-kernel shapes need no GEMM workspace; decode shapes may (split K)
    assert L.nvfp4_gemm_workspace_size(8192, 4096, 4096) == 0
    assert L.bf16_gemm_workspace_size(8192, 4096, 4096) == 0
    assert L.nvfp4_gemm_workspace_size(0, 4096, 4096) == 0
    for f in (L.nvfp4_gemm_workspace_size, L.bf16_gemm_workspace_size):
        for M in (1, 8, 64):
            ws = f(M, 4096, 4096)
            assert ws == 0 or ws % (M * 4096 * 4) == 0  # S slices of FP32 [M, N]


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_quantize_argument_errors(L):
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EINVAL, NVFP4_EWORKSPACE, NVFP4_OK

    q = L.nvfp4_quantize
    assert q(FAKE, 4, 24, 24, FAKE, FAKE, FAKE, 0, FAKE, 4096, None) == NVFP4_EINVAL  # cols % 16
    assert b"multiple of 16" in L.nvfp4_last_error()
    assert q(None, 4, 32, 32, FAKE, FAKE, FAKE, 1, None, 0, None) == NVFP4_EINVAL  # null x
    assert q(FAKE, 4, 32, 16, FAKE, FAKE, FAKE, 1, None, 0, None) == NVFP4_EINVAL  # ld < cols
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, FAKE, 7, None, 0, None) == NVFP4_EINVAL  # alpha mode
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, FAKE, 0, None, 0, None) == NVFP4_EWORKSPACE
    assert q(ctypes.c_void_p(0x1008), 4, 32, 32, FAKE, FAKE, FAKE, 1, None, 0, None) == NVFP4_EINVAL  # align
    assert q(None, 0, 32, 32, None, None, None, 0, None, 0, None) == NVFP4_OK  # empty: no launch
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EUNSUPPORTED

    big = 1 << 30  # past the kernels' 32-bit row indexing
    assert q(FAKE, 1, big, big, FAKE, FAKE, FAKE, 1, None, 0, None) == NVFP4_EUNSUPPORTED
    assert b"2^30" in L.nvfp4_last_error()
    assert q(FAKE, 1 << 31, 16, 16, FAKE, FAKE, FAKE, 1, None, 0, None) == NVFP4_EUNSUPPORTED  # items


def test_gemm_argument_errors(L):
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_OK

    g = L.nvfp4_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 24, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL  # K % 16
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 5, 8, None, 0, None) == NVFP4_EINVAL  # dtype
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 4, None, 0, None) == NVFP4_EINVAL  # ld_out
    assert g(FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL  # null alpha
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 32, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL
    assert g(None, None, None, None, None, None, 0, 8, 32, None, 0, 8, None, 0, None) == NVFP4_OK
    q = L.nvfp4_gemm_quant_out
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 24, 32, FAKE, FAKE, FAKE, None) == NVFP4_EINVAL  # N % 16
    assert b"multiple of 16" in L.nvfp4_last_error()
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 32, FAKE, FAKE, None, None) == NVFP4_EINVAL  # y_alpha
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 32, ctypes.c_void_p(0x1002), FAKE, FAKE, None) == NVFP4_EINVAL
    assert q(None, None, None, None, None, None, 0, 16, 32, None, None, None, None) == NVFP4_OK
    odd = ctypes.c_void_p(0x1002)
    assert g(FAKE, odd, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL  # scale align
    assert b"4-byte aligned" in L.nvfp4_last_error()
    b = L.bf16_gemm
    assert b(FAKE, FAKE, 8, 8, 12, FAKE, 0, 8, None, 0, None) == NVFP4_EUNSUPPORTED  # K % 8
    assert b(None, FAKE, 8, 8, 16, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL
    f = L.nvfp4_quant_gemm
    assert f(FAKE, 32, FAKE, 0, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == -4  # workspace
    assert f(FAKE, 16, FAKE, 1, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL  # ld_x
    misaligned = ctypes.c_void_p(0x1008)  # workspaces hold uint32 / float partials and 16-byte code rows
    assert f(FAKE, 32, FAKE, 0, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, misaligned, 4096, None) == NVFP4_EINVAL
    assert b"workspace must be 16-byte aligned" in L.nvfp4_last_error()
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, misaligned, 4096, None) == NVFP4_EINVAL
    assert b"workspace must be 16-byte aligned" in L.nvfp4_last_error()
    assert b(FAKE, FAKE, 8, 8, 16, FAKE, 0, 8, misaligned, 4096, None) == NVFP4_EINVAL
    assert b"workspace must be 16-byte aligned" in L.nvfp4_last_error()


def test_quant_out_dynamic_argument_errors(L):
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EINVAL, NVFP4_EWORKSPACE

    f = L.nvfp4_gemm_quant_out_dynamic
    need = L.nvfp4_gemm_quant_out_dynamic_workspace_size(64, 256, 512)
    assert need >= 64 * 256 * 4  # the FP32 product
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert f(*args, 64, 264, 512, FAKE, FAKE, FAKE, FAKE, need, None) == NVFP4_EINVAL  # N % 16
    assert b"multiple of 16" in L.nvfp4_last_error()
    assert f(*args, 64, 256, 520, FAKE, FAKE, FAKE, FAKE, need, None) == NVFP4_EINVAL  # K % 16
    assert f(*args, 64, 256, 512, None, FAKE, FAKE, FAKE, need, None) == NVFP4_EINVAL  # null y_codes
    assert f(*args, 64, 256, 512, FAKE, FAKE, FAKE, FAKE, need - 1, None) == NVFP4_EWORKSPACE
    assert f(*args, 64, 256, 512, FAKE, FAKE, FAKE, None, 0, None) == NVFP4_EWORKSPACE
    assert f(*args, 64, 256, 512, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1010), need, None) == NVFP4_EINVAL  # alignment
    assert b"256-byte" in L.nvfp4_last_error()


def test_decode_packed_argument_errors(L):
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_EWORKSPACE, NVFP4_OK

    assert L.nvfp4_decode_pack_size(1000, 4096) == 63 * 32 * 1152
    assert L.nvfp4_decode_pack_size(1000, 4160) == 0 and L.nvfp4_decode_pack_size(0, 4096) == 0
    p = L.nvfp4_decode_pack
    assert p(FAKE, FAKE, 64, 4160, FAKE, None) == NVFP4_EUNSUPPORTED  # K % 128
    assert b"multiple of 128" in L.nvfp4_last_error()
    assert p(None, FAKE, 64, 4096, FAKE, None) == NVFP4_EINVAL
    assert p(FAKE, FAKE, 64, 4096, ctypes.c_void_p(0x1008), None) == NVFP4_EINVAL  # packed alignment
    assert p(None, None, 0, 4096, None, None) == NVFP4_OK  # empty: no launch
    g = L.nvfp4_gemm_packed
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    assert g(*args, 65, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EUNSUPPORTED  # decode batches only
    assert b"decode batches" in L.nvfp4_last_error()
    assert g(*args, 8, 64, 4160, FAKE, 0, 64, None, 0, None) == NVFP4_EUNSUPPORTED  # K % 128
    assert g(FAKE, FAKE, FAKE, None, FAKE, 8, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EINVAL  # no weight
    assert g(*args, 8, 64, 4096, FAKE, 0, 32, None, 0, None) == NVFP4_EINVAL  # ld_out < N
    assert g(*args, -1, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EINVAL
    assert g(None, None, None, None, None, 0, 64, 4096, None, 0, 64, None, 0, None) == NVFP4_OK
    q = L.nvfp4_quant_gemm_packed
    qa = (FAKE, 4096, FAKE)
    assert q(*qa, 0, FAKE, FAKE, 65, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EUNSUPPORTED
    assert q(*qa, 3, FAKE, FAKE, 8, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EINVAL  # alpha mode
    # batch 32 takes the quantizer into the workspace: without one, EWORKSPACE
    assert q(*qa, 0, FAKE, FAKE, 32, 4096, 4096, FAKE, 0, 4096, None, 0, None) == NVFP4_EWORKSPACE
    # one row takes the fused kernel, whose dynamic alpha needs the amax partials
    assert q(*qa, 0, FAKE, FAKE, 1, 4096, 4096, FAKE, 0, 4096, None, 0, None) == NVFP4_EWORKSPACE
    assert q((FAKE), 4000, FAKE, 0, FAKE, FAKE, 8, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EINVAL  # ld_x


def test_bf16_packed_argument_errors(L):
    from nvfp4_prefill_gemm_amd.binding import NVFP4_EINVAL, NVFP4_EUNSUPPORTED, NVFP4_OK

    assert L.bf16_decode_pack_size(1000, 4096) == 63 * 128 * 1024
    assert L.bf16_decode_pack_size(1000, 4104) == 0
    p = L.bf16_decode_pack
    assert p(FAKE, 64, 4104, FAKE, None) == NVFP4_EUNSUPPORTED  # K % 32
    assert p(None, 64, 4096, FAKE, None) == NVFP4_EINVAL
    assert p(FAKE, 64, 4096, ctypes.c_void_p(0x1008), None) == NVFP4_EINVAL
    assert p(None, 0, 4096, None, None) == NVFP4_OK
    g = L.bf16_gemm_packed
    assert g(FAKE, FAKE, 65, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EUNSUPPORTED
    assert g(FAKE, FAKE, 8, 64, 4104, FAKE, 0, 64, None, 0, None) == NVFP4_EUNSUPPORTED
    assert g(FAKE, None, 8, 64, 4096, FAKE, 0, 64, None, 0, None) == NVFP4_EINVAL
    assert g(FAKE, FAKE, 8, 64, 4096, FAKE, 0, 32, None, 0, None) == NVFP4_EINVAL  # ld_out
    assert g(FAKE, FAKE, 8, 64, 4096, FAKE, 0, 64, ctypes.c_void_p(0x1008), 4096, None) == NVFP4_EINVAL
    assert g(None, None, 0, 64, 4096, None, 0, 64, None, 0, None) == NVFP4_OK
