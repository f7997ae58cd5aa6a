// Internal launch interface shared by the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace nvfp4 {

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device and process (`done` holds one bit per device id below 32;
// devices beyond that set it on every call).  The attribute is per device, so
// a process that drives several GPUs sets it on each.
inline hipError_t set_dyn_lds_once(std::atomic<uint32_t> &done, const void *kern, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint32_t bit = dev >= 0 && dev < 32 ? 1u << dev : 0u;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

// Number of per-workgroup partial maxima the amax pass writes for a tensor.
int amax_parts(int64_t rows, int64_t cols);

hipError_t launch_amax_partials(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                                uint32_t *partials, int nparts, hipStream_t s);

// dynamic != 0: alpha = max(partials[0..nparts)) / 2688 is written to *alpha.
hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint8_t *scales, float *alpha, int dynamic, const uint32_t *partials,
                           int nparts, hipStream_t s);

// alpha from partials only (fused path, dynamic mode).
hipError_t launch_alpha_from_partials(const uint32_t *partials, int nparts, float *alpha, hipStream_t s);

enum OutType { OUT_F32 = 0, OUT_BF16 = 1, OUT_NVFP4 = 2 };

hipError_t launch_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                             int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                             hipStream_t s);

// Tile GEMM whose epilogue quantizes Y to NVFP4 with a static tensor scale
// (codes [M, N/2], scales [M, N/16]); N % 16 == 0, y_codes 4-byte aligned.
hipError_t launch_gemm_nvfp4_quant_out(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                       const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                       int64_t M, int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales,
                                       const float *y_alpha, hipStream_t s);

hipError_t launch_gemm_fused(const uint16_t *x, int64_t ld_x, const float *a_alpha,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                             int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                             hipStream_t s);

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                            void *out, int out_type, int64_t ld_out, hipStream_t s);

hipError_t launch_skinny_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                              void *out, int out_type, int64_t ld_out, hipStream_t s);

// NVFP4 x NVFP4 at decode shapes: M <= kSkinnyMaxM, K % 32 == 0, codes
// 16-byte and scales 2-byte aligned (nvfp4_gemm checks and otherwise uses the
// tile kernel).
hipError_t launch_skinny_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                               int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                               hipStream_t s);

// Fused decode (BF16 activations quantized into LDS by every workgroup):
// M <= 16, M * K <= kFusedDecodeMaxElems, K % 32 == 0, x rows 16-byte
// aligned; dynamic != 0 computes alpha_A in every workgroup.
hipError_t launch_skinny_fused(const uint16_t *x, int64_t ld_x, float *a_alpha, int dynamic,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                               int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                               hipStream_t s);

// nvfp4_quant_gemm routes M <= kFusedDecodeMaxM with M * K <=
// kFusedDecodeMaxElems (108 KB of codes and scales in LDS: every Qwen3-8B
// layer at 16 tokens) to the fused decode kernel.
constexpr int64_t kFusedDecodeMaxM = 16;
constexpr int64_t kFusedDecodeMaxElems = 16 * 12288;

// Largest M routed to the skinny decode kernels by bf16_gemm and nvfp4_gemm.
constexpr int64_t kSkinnyMaxM = 64;
// The decode kernels address each operand through a buffer resource of fewer
// than 2^31 bytes (64 rows of BF16), so they take K < kSkinnyMaxK.
constexpr int64_t kSkinnyMaxK = int64_t(1) << 24;

hipError_t launch_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                              uint8_t *scales, hipStream_t s);

hipError_t launch_mx_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                          const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                          int64_t ld_out, hipStream_t s);

hipError_t launch_fill_zero(void *out, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s);

}  // namespace nvfp4
