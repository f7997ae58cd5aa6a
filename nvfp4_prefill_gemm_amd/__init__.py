"""MI355X-native NVFP4 prefill GEMM path: gfx950 HIP kernels behind a C ABI.

The kernels live in ``libnvfp4.so`` (built from ``csrc/`` by ``build.py``);
``binding`` exposes the C entry points under the same names.  ``workloads``
holds the seeded synthetic inputs.
"""
from . import workloads  # noqa: F401


def __getattr__(name):
    # the binding imports torch; load it on first use of an entry point
    if name in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_quant_gemm", "nvfp4_gemm_quant_out",
                "nvfp4_gemm_quant_out_dynamic", "nvfp4_decode_pack", "nvfp4_gemm_packed",
                "nvfp4_quant_gemm_packed", "bf16_gemm", "bf16_decode_pack", "bf16_gemm_packed",
                "mxfp4_quantize", "mxfp4_gemm",
                "binding", "lib", "last_error"):
        import importlib

        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
