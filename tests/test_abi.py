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
              "nvfp4_abi_version", "nvfp4_quantize_workspace_size", "nvfp4_quant_gemm_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_abi_version(L):
    assert L.nvfp4_abi_version() == 1


def test_workspace_sizes(L):
    assert L.nvfp4_quantize_workspace_size(0, 4096) == 0
    assert L.nvfp4_quantize_workspace_size(8192, 4096) > 0
    assert L.nvfp4_quantize_workspace_size(8192, 4096) <= 4096
    assert L.nvfp4_quant_gemm_workspace_size(128, 256) == L.nvfp4_quantize_workspace_size(128, 256)


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
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 24, FAKE, 0, 8, None) == NVFP4_EINVAL  # K % 16
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 5, 8, None) == NVFP4_EINVAL  # dtype
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 4, None) == NVFP4_EINVAL  # ld_out
    assert g(FAKE, FAKE, None, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None) == NVFP4_EINVAL  # null alpha
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 32, FAKE, 0, 8, None) == NVFP4_EINVAL
    assert g(None, None, None, None, None, None, 0, 8, 32, None, 0, 8, None) == NVFP4_OK
    q = L.nvfp4_gemm_quant_out
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 24, 32, FAKE, FAKE, FAKE, None) == NVFP4_EINVAL  # N % 16
    assert b"multiple of 16" in L.nvfp4_last_error()
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 32, FAKE, FAKE, None, None) == NVFP4_EINVAL  # y_alpha
    assert q(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 32, ctypes.c_void_p(0x1002), FAKE, FAKE, None) == NVFP4_EINVAL
    assert q(None, None, None, None, None, None, 0, 16, 32, None, None, None, None) == NVFP4_OK
    odd = ctypes.c_void_p(0x1002)
    assert g(FAKE, odd, FAKE, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None) == NVFP4_EINVAL  # scale align
    assert b"4-byte aligned" in L.nvfp4_last_error()
    b = L.bf16_gemm
    assert b(FAKE, FAKE, 8, 8, 12, FAKE, 0, 8, None) == NVFP4_EUNSUPPORTED  # K % 8
    assert b(None, FAKE, 8, 8, 16, FAKE, 0, 8, None) == NVFP4_EINVAL
    f = L.nvfp4_quant_gemm
    assert f(FAKE, 32, FAKE, 0, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == -4  # workspace
    assert f(FAKE, 16, FAKE, 1, FAKE, FAKE, FAKE, 8, 8, 32, FAKE, 0, 8, None, 0, None) == NVFP4_EINVAL  # ld_x
