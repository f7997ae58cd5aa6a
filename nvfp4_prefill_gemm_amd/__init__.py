"""MI355X-native NVFP4 prefill GEMM path (gfx950 HIP kernels behind a C ABI)."""
