// C ABI of the NVFP4 prefill GEMM library: argument checks, then dispatch to
// the gfx950 kernels on the caller's stream.  Nothing here allocates device
// memory or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/nvfp4.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return NVFP4_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int check_out(const void *out, int out_dtype, int64_t N, int64_t ld_out, const char *fn) {
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_EINVAL, "%s: out_dtype must be NVFP4_OUT_F32 or NVFP4_OUT_BF16", fn);
    if (!out) return fail(NVFP4_EINVAL, "%s: out is null", fn);
    if (ld_out < N) return fail(NVFP4_EINVAL, "%s: ld_out (%lld) < N (%lld)", fn, (long long)ld_out, (long long)N);
    if (!aligned(out, out_dtype == NVFP4_OUT_F32 ? 4 : 2)) return fail(NVFP4_EINVAL, "%s: out is misaligned", fn);
    return NVFP4_OK;
}

int check_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *alpha, const char *which, const char *fn) {
    if (!codes || !scales || !alpha) return fail(NVFP4_EINVAL, "%s: %s codes, scales and alpha must be non-null", fn, which);
    if (!aligned(codes, 16)) return fail(NVFP4_EINVAL, "%s: %s codes must be 16-byte aligned", fn, which);
    if (!aligned(scales, 4)) return fail(NVFP4_EINVAL, "%s: %s scales must be 4-byte aligned", fn, which);
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char *nvfp4_last_error(void) { return g_err; }

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)nvfp4::amax_parts(rows, cols) * sizeof(uint32_t);
}

int nvfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes, uint8_t *scales,
                   float *alpha, int alpha_mode, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "nvfp4_quantize";
    if (rows < 0 || cols < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (cols % 16 != 0) return fail(NVFP4_EINVAL, "%s: cols (%lld) must be a multiple of 16", fn, (long long)cols);
    if (alpha_mode != NVFP4_ALPHA_DYNAMIC && alpha_mode != NVFP4_ALPHA_STATIC)
        return fail(NVFP4_EINVAL, "%s: bad alpha_mode %d", fn, alpha_mode);
    if (rows == 0 || cols == 0) return ok();
    if (!x_bf16 || !codes || !scales || !alpha) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (ld_x < cols || ld_x % 8 != 0) return fail(NVFP4_EINVAL, "%s: ld_x must be >= cols and a multiple of 8", fn);
    if (!aligned(x_bf16, 16)) return fail(NVFP4_EINVAL, "%s: x must be 16-byte aligned", fn);
    if (!aligned(codes, 16)) return fail(NVFP4_EINVAL, "%s: codes must be 16-byte aligned", fn);
    if (!aligned(alpha, 4)) return fail(NVFP4_EINVAL, "%s: alpha is misaligned", fn);
    if (cols >= (int64_t(1) << 30) || rows * ((cols + 2047) / 2048) >= (int64_t(1) << 31))
        return fail(NVFP4_EUNSUPPORTED, "%s: cols must be < 2^30 and rows * ceil(cols / 2048) < 2^31", fn);
    hipStream_t s = as_stream(stream);
    const int dyn = alpha_mode == NVFP4_ALPHA_DYNAMIC;
    const int nparts = nvfp4::amax_parts(rows, cols);
    if (dyn) {
        const size_t need = (size_t)nparts * sizeof(uint32_t);
        if (!workspace || workspace_bytes < need)
            return fail(NVFP4_EWORKSPACE, "%s: dynamic alpha needs %zu workspace bytes", fn, need);
        if (!aligned(workspace, 4)) return fail(NVFP4_EINVAL, "%s: workspace is misaligned", fn);
        int rc = hip_status(nvfp4::launch_amax_partials((const uint16_t *)x_bf16, rows, cols, ld_x,
                                                        (uint32_t *)workspace, nparts, s),
                            "amax kernel");
        if (rc) return rc;
    }
    return hip_status(nvfp4::launch_quantize((const uint16_t *)x_bf16, rows, cols, ld_x, codes, scales, alpha, dyn,
                                             (const uint32_t *)workspace, nparts, s),
                      "quantize kernel");
}

int nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha, const uint8_t *w_codes,
               const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K, void *out,
               int out_dtype, int64_t ld_out, void *stream) {
    const char *fn = "nvfp4_gemm";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
    if (M == 0 || N == 0) return ok();
    int rc = check_out(out, out_dtype, N, ld_out, fn);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if ((rc = check_nvfp4(a_codes, a_scales, a_alpha, "A", fn))) return rc;
    if ((rc = check_nvfp4(w_codes, w_scales, w_alpha, "W", fn))) return rc;
    if (M <= nvfp4::kSkinnyMaxM && K < nvfp4::kSkinnyMaxK && K % 32 == 0)
        return hip_status(nvfp4::launch_skinny_nvfp4(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K,
                                                     out, out_dtype, ld_out, s),
                          "nvfp4 decode kernel");
    return hip_status(nvfp4::launch_gemm_nvfp4(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out,
                                               out_dtype, ld_out, s),
                      "nvfp4 gemm kernel");
}

int nvfp4_gemm_quant_out(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                         const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                         int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales, const float *y_alpha,
                         void *stream) {
    const char *fn = "nvfp4_gemm_quant_out";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
    if (N % 16 != 0) return fail(NVFP4_EINVAL, "%s: N (%lld) must be a multiple of 16", fn, (long long)N);
    if (M == 0 || N == 0) return ok();
    if (!y_codes || !y_scales || !y_alpha) return fail(NVFP4_EINVAL, "%s: null output pointer", fn);
    if (!aligned(y_codes, 4)) return fail(NVFP4_EINVAL, "%s: y_codes must be 4-byte aligned", fn);
    hipStream_t s = as_stream(stream);
    int rc;
    if (K == 0) {  // Y = 0: zero codes and zero scales
        if ((rc = hip_status(nvfp4::launch_fill_zero(y_codes, M, N / 2, N / 2, 1, s), "fill kernel"))) return rc;
        return hip_status(nvfp4::launch_fill_zero(y_scales, M, N / 16, N / 16, 1, s), "fill kernel");
    }
    if ((rc = check_nvfp4(a_codes, a_scales, a_alpha, "A", fn))) return rc;
    if ((rc = check_nvfp4(w_codes, w_scales, w_alpha, "W", fn))) return rc;
    return hip_status(nvfp4::launch_gemm_nvfp4_quant_out(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N,
                                                         K, y_codes, y_scales, y_alpha, s),
                      "nvfp4 gemm kernel (quantized output)");
}

size_t nvfp4_quant_gemm_workspace_size(int64_t M, int64_t K) { return nvfp4_quantize_workspace_size(M, K); }

int nvfp4_quant_gemm(const void *x_bf16, int64_t ld_x, float *a_alpha, int alpha_mode, const uint8_t *w_codes,
                     const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K, void *out,
                     int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "nvfp4_quant_gemm";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
    if (alpha_mode != NVFP4_ALPHA_DYNAMIC && alpha_mode != NVFP4_ALPHA_STATIC)
        return fail(NVFP4_EINVAL, "%s: bad alpha_mode %d", fn, alpha_mode);
    if (M == 0 || N == 0) return ok();
    int rc = check_out(out, out_dtype, N, ld_out, fn);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if (!x_bf16 || !a_alpha) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (ld_x < K || ld_x % 8 != 0) return fail(NVFP4_EINVAL, "%s: ld_x must be >= K and a multiple of 8", fn);
    if (!aligned(x_bf16, 16)) return fail(NVFP4_EINVAL, "%s: x must be 16-byte aligned", fn);
    if ((rc = check_nvfp4(w_codes, w_scales, w_alpha, "W", fn))) return rc;
    if (alpha_mode == NVFP4_ALPHA_DYNAMIC) {
        const int nparts = nvfp4::amax_parts(M, K);
        const size_t need = (size_t)nparts * sizeof(uint32_t);
        if (!workspace || workspace_bytes < need)
            return fail(NVFP4_EWORKSPACE, "%s: dynamic alpha needs %zu workspace bytes", fn, need);
    }
    if (M <= nvfp4::kFusedDecodeMaxM && M * K <= nvfp4::kFusedDecodeMaxElems && K % 32 == 0)
        return hip_status(nvfp4::launch_skinny_fused((const uint16_t *)x_bf16, ld_x, a_alpha,
                                                     alpha_mode == NVFP4_ALPHA_DYNAMIC, w_codes, w_scales, w_alpha, M,
                                                     N, K, out, out_dtype, ld_out, s),
                          "fused decode kernel");
    if (alpha_mode == NVFP4_ALPHA_DYNAMIC) {
        const int nparts = nvfp4::amax_parts(M, K);
        if ((rc = hip_status(nvfp4::launch_amax_partials((const uint16_t *)x_bf16, M, K, ld_x, (uint32_t *)workspace,
                                                         nparts, s),
                             "amax kernel")))
            return rc;
        if ((rc = hip_status(nvfp4::launch_alpha_from_partials((const uint32_t *)workspace, nparts, a_alpha, s),
                             "alpha kernel")))
            return rc;
    }
    return hip_status(nvfp4::launch_gemm_fused((const uint16_t *)x_bf16, ld_x, a_alpha, w_codes, w_scales, w_alpha, M,
                                               N, K, out, out_dtype, ld_out, s),
                      "fused gemm kernel");
}

int bf16_gemm(const void *a_bf16, const void *w_bf16, int64_t M, int64_t N, int64_t K, void *out, int out_dtype,
              int64_t ld_out, void *stream) {
    const char *fn = "bf16_gemm";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 8 != 0) return fail(NVFP4_EUNSUPPORTED, "%s: K (%lld) must be a multiple of 8", fn, (long long)K);
    if (M == 0 || N == 0) return ok();
    int rc = check_out(out, out_dtype, N, ld_out, fn);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if (!a_bf16 || !w_bf16) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (!aligned(a_bf16, 16) || !aligned(w_bf16, 16)) return fail(NVFP4_EINVAL, "%s: A and W must be 16-byte aligned", fn);
    if (M <= nvfp4::kSkinnyMaxM && K < nvfp4::kSkinnyMaxK)
        return hip_status(nvfp4::launch_skinny_bf16((const uint16_t *)a_bf16, (const uint16_t *)w_bf16, M, N, K, out,
                                                    out_dtype, ld_out, s),
                          "skinny bf16 kernel");
    return hip_status(nvfp4::launch_gemm_bf16((const uint16_t *)a_bf16, (const uint16_t *)w_bf16, M, N, K, out,
                                              out_dtype, ld_out, s),
                      "bf16 gemm kernel");
}

int mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes, uint8_t *scales,
                   void *stream) {
    const char *fn = "mxfp4_quantize";
    if (rows < 0 || cols < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (cols % 32 != 0) return fail(NVFP4_EINVAL, "%s: cols (%lld) must be a multiple of 32", fn, (long long)cols);
    if (rows == 0 || cols == 0) return ok();
    if (!x_bf16 || !codes || !scales) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (ld_x < cols || ld_x % 8 != 0) return fail(NVFP4_EINVAL, "%s: ld_x must be >= cols and a multiple of 8", fn);
    if (!aligned(x_bf16, 16) || !aligned(codes, 16)) return fail(NVFP4_EINVAL, "%s: x and codes must be 16-byte aligned", fn);
    return hip_status(nvfp4::launch_mx_quantize((const uint16_t *)x_bf16, rows, cols, ld_x, codes, scales,
                                                as_stream(stream)),
                      "mx quantize kernel");
}

int mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes, const uint8_t *w_scales,
               int64_t M, int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out, void *stream) {
    const char *fn = "mxfp4_gemm";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 32 != 0) return fail(NVFP4_EINVAL, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
    if (M == 0 || N == 0) return ok();
    int rc = check_out(out, out_dtype, N, ld_out, fn);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if (!a_codes || !a_scales || !w_codes || !w_scales) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 8) || !aligned(w_scales, 8))
        return fail(NVFP4_EINVAL, "%s: codes must be 16-byte and scales 8-byte aligned", fn);
    return hip_status(nvfp4::launch_mx_gemm(a_codes, a_scales, w_codes, w_scales, M, N, K, out, out_dtype, ld_out, s),
                      "mx gemm kernel");
}

}  // extern "C"
