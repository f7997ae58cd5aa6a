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

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

bool decode_shape(int64_t M, int64_t K, int kmult) {
    return M <= nvfp4::kSkinnyMaxM && K < nvfp4::kSkinnyMaxK && K % kmult == 0;
}

// nvfp4_quant_gemm's workspace when it quantizes into the workspace and then
// runs the NVFP4 GEMM: codes [M, K/2], scales [M, K/16] (or, for the decode
// kernel's batches of more than two rows with K % 128 == 0, both in its
// packed block layout at `codes`), the amax partials (dynamic alpha) and the
// GEMM's split-K partials, each 256-byte aligned.
struct QgLayout {
    size_t codes, scales, parts, split, total;
    bool pack_a;
};
QgLayout qg_layout(int64_t M, int64_t N, int64_t K, bool dyn) {
    QgLayout l;
    l.codes = 0;
    l.pack_a = decode_shape(M, K, 32) && nvfp4::decode_pack_a_route(M, K);
    if (l.pack_a) {
        l.scales = align256(nvfp4::decode_pack_a_bytes(M, K));
        l.parts = l.scales;
    } else {
        l.scales = align256((size_t)M * (size_t)(K / 2));
        l.parts = l.scales + align256((size_t)M * (size_t)(K / 16));
    }
    l.split = l.parts + (dyn ? align256((size_t)nvfp4::amax_parts(M, K) * sizeof(uint32_t)) : 0);
    size_t split_bytes = 0;
    if (M <= nvfp4::kSkinnyMaxM && K < nvfp4::kSkinnyMaxK && K % 32 == 0)
        split_bytes = nvfp4::decode_workspace_bytes(nvfp4::DECODE_NVFP4, M, N, K);
    l.total = l.split + split_bytes;
    return l;
}

bool fused_decode_shape(int64_t M, int64_t N, int64_t K) { return nvfp4::fused_decode_route(M, N, K); }


int quantize_impl(const char *fn, const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                  uint8_t *scales, float *alpha, int alpha_mode, void *workspace, size_t workspace_bytes,
                  bool use_scratch, void *stream) {
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
    if (dyn && use_scratch) {
        uint32_t *p = nullptr;
        size_t bytes = 0;
        if (int rc = hip_status(nvfp4::quantize_scratch(&p, &bytes), "scratch lookup")) return rc;
        if ((size_t)nparts * sizeof(uint32_t) > bytes)
            return fail(NVFP4_EUNSUPPORTED, "%s: %d amax partials exceed the %zu-byte scratch", fn, nparts, bytes);
        workspace = p;
        workspace_bytes = bytes;
    }
    if (dyn) {
        const size_t need = (size_t)nparts * sizeof(uint32_t);
        if (!workspace || workspace_bytes < need)
            return fail(NVFP4_EWORKSPACE, "%s: dynamic alpha needs %zu workspace bytes", fn, need);
        if (!aligned(workspace, 4)) return fail(NVFP4_EINVAL, "%s: workspace is misaligned", fn);
        return hip_status(nvfp4::launch_quantize_dynamic((const uint16_t *)x_bf16, rows, cols, ld_x, codes, scales,
                                                         alpha, (uint32_t *)workspace, nparts, s),
                          "quantize kernel");
    }
    return hip_status(nvfp4::launch_quantize((const uint16_t *)x_bf16, rows, cols, ld_x, codes, scales, alpha, dyn,
                                             (const uint32_t *)workspace, nparts, s),
                      "quantize kernel");
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
    return quantize_impl("nvfp4_quantize", x_bf16, rows, cols, ld_x, codes, scales, alpha, alpha_mode, workspace,
                         workspace_bytes, false, stream);
}

int nvfp4_quantize_noalloc(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                           uint8_t *scales, float *alpha, int alpha_mode, void *stream) {
    return quantize_impl("nvfp4_quantize_noalloc", x_bf16, rows, cols, ld_x, codes, scales, alpha, alpha_mode,
                         nullptr, 0, true, stream);
}

size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || !decode_shape(M, K, 32)) return 0;
    return nvfp4::decode_workspace_bytes(nvfp4::DECODE_NVFP4, M, N, K);
}

int nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha, const uint8_t *w_codes,
               const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K, void *out,
               int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream) {
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
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    if (decode_shape(M, K, 32))
        return hip_status(nvfp4::launch_skinny_nvfp4(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K,
                                                     out, out_dtype, ld_out, workspace, workspace_bytes, s),
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

size_t nvfp4_gemm_quant_out_dynamic_workspace_size(int64_t M, int64_t N, int64_t K) {
    (void)K;
    if (M <= 0 || N <= 0) return 0;
    return align256((size_t)M * (size_t)N * sizeof(float)) +
           align256((size_t)nvfp4::gemm_amax_parts_bound(M, N) * sizeof(uint32_t));
}

int nvfp4_gemm_quant_out_dynamic(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                 const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                                 int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales, float *y_alpha,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "nvfp4_gemm_quant_out_dynamic";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 16 != 0) return fail(NVFP4_EINVAL, "%s: K (%lld) must be a multiple of 16", fn, (long long)K);
    if (N % 16 != 0) return fail(NVFP4_EINVAL, "%s: N (%lld) must be a multiple of 16", fn, (long long)N);
    if (M == 0 || N == 0) return ok();
    if (!y_codes || !y_scales || !y_alpha) return fail(NVFP4_EINVAL, "%s: null output pointer", fn);
    if (!aligned(y_codes, 4)) return fail(NVFP4_EINVAL, "%s: y_codes must be 4-byte aligned", fn);
    if (!aligned(y_alpha, 4)) return fail(NVFP4_EINVAL, "%s: y_alpha is misaligned", fn);
    hipStream_t s = as_stream(stream);
    int rc;
    if (K == 0) {  // Y = 0: alpha 0, zero codes and zero scales
        if ((rc = hip_status(nvfp4::launch_fill_zero(y_alpha, 1, 1, 1, 4, s), "fill kernel"))) return rc;
        if ((rc = hip_status(nvfp4::launch_fill_zero(y_codes, M, N / 2, N / 2, 1, s), "fill kernel"))) return rc;
        return hip_status(nvfp4::launch_fill_zero(y_scales, M, N / 16, N / 16, 1, s), "fill kernel");
    }
    if ((rc = check_nvfp4(a_codes, a_scales, a_alpha, "A", fn))) return rc;
    if ((rc = check_nvfp4(w_codes, w_scales, w_alpha, "W", fn))) return rc;
    const size_t need = nvfp4_gemm_quant_out_dynamic_workspace_size(M, N, K);
    if (!workspace || workspace_bytes < need)
        return fail(NVFP4_EWORKSPACE, "%s: needs %zu bytes of workspace, got %zu", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(NVFP4_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    const int64_t nparts = nvfp4::gemm_amax_parts(M, N);
    if (nparts > 0x7FFFFFFF) return fail(NVFP4_EUNSUPPORTED, "%s: too many output tiles", fn);
    float *y = (float *)workspace;
    uint32_t *parts = (uint32_t *)((char *)workspace + align256((size_t)M * (size_t)N * sizeof(float)));
    if ((rc = hip_status(nvfp4::launch_gemm_nvfp4_f32_amax(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M,
                                                           N, K, y, parts, s),
                         "nvfp4 gemm kernel (FP32 output and amax)")))
        return rc;
    if ((rc = hip_status(nvfp4::launch_alpha_from_partials(parts, (int)nparts, y_alpha, s), "alpha kernel")))
        return rc;
    return hip_status(nvfp4::launch_quantize_f32(y, M, N, N, y_codes, y_scales, y_alpha, s), "FP32 quantize kernel");
}

size_t nvfp4_quant_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const size_t parts = nvfp4_quantize_workspace_size(M, K);  // the minimum with a dynamic alpha
    if (fused_decode_shape(M, N, K)) {
        const size_t split = nvfp4::decode_workspace_bytes(nvfp4::DECODE_FUSED, M, N, K);
        return split > parts ? split : parts;
    }
    return qg_layout(M, N, K, true).total;
}

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
    const bool dyn = alpha_mode == NVFP4_ALPHA_DYNAMIC;
    if (dyn) {
        const int nparts = nvfp4::amax_parts(M, K);
        const size_t need = (size_t)nparts * sizeof(uint32_t);
        if (!workspace || workspace_bytes < need)
            return fail(NVFP4_EWORKSPACE, "%s: dynamic alpha needs %zu workspace bytes", fn, need);
    }
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    // decode batches: one kernel quantizes the batch into LDS and runs the decode GEMM
    if (fused_decode_shape(M, N, K))
        return hip_status(nvfp4::launch_skinny_fused((const uint16_t *)x_bf16, ld_x, a_alpha, dyn, w_codes, w_scales,
                                                     w_alpha, M, N, K, out, out_dtype, ld_out, workspace,
                                                     workspace_bytes, s),
                          "fused decode kernel");
    // otherwise quantize once into the workspace and run the NVFP4 GEMM: the
    // tile kernel's in-prologue quantization repeats for every column tile
    // and measured slower at every prefill size
    const QgLayout l = qg_layout(M, N, K, dyn);
    uint8_t *wsb = (uint8_t *)workspace;
    if (workspace && workspace_bytes >= l.split) {
        uint8_t *codes = wsb + l.codes, *scales = wsb + l.scales;
        const int nparts = nvfp4::amax_parts(M, K);
        if ((rc = hip_status(dyn ? nvfp4::launch_quantize_dynamic((const uint16_t *)x_bf16, M, K, ld_x, codes, scales,
                                                                  a_alpha, (uint32_t *)(wsb + l.parts), nparts, s,
                                                                  l.pack_a)
                                 : nvfp4::launch_quantize((const uint16_t *)x_bf16, M, K, ld_x, codes, scales, a_alpha,
                                                          0, nullptr, nparts, s, l.pack_a),
                             "quantize kernel")))
            return rc;
        if (decode_shape(M, K, 32))
            return hip_status(nvfp4::launch_skinny_nvfp4(codes, scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K,
                                                         out, out_dtype, ld_out, wsb + l.split,
                                                         workspace_bytes - l.split, s,
                                                         l.pack_a ? nvfp4::kPackA : 0),
                              "nvfp4 decode kernel");
        return hip_status(nvfp4::launch_gemm_nvfp4(codes, scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out,
                                                   out_dtype, ld_out, s),
                          "nvfp4 gemm kernel");
    }
    // a workspace too small for the quantized activations: the tile kernel
    // quantizes in its operand staging
    if (dyn) {
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

size_t bf16_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || !decode_shape(M, K, 8)) return 0;
    return nvfp4::decode_workspace_bytes(nvfp4::DECODE_BF16, M, N, K);
}

int bf16_gemm(const void *a_bf16, const void *w_bf16, int64_t M, int64_t N, int64_t K, void *out, int out_dtype,
              int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream) {
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
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    if (decode_shape(M, K, 8))
        return hip_status(nvfp4::launch_skinny_bf16((const uint16_t *)a_bf16, (const uint16_t *)w_bf16, M, N, K, out,
                                                    out_dtype, ld_out, workspace, workspace_bytes, s),
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

size_t nvfp4_decode_pack_size(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 128 != 0) return 0;
    return (size_t)((N + 15) / 16) * (size_t)(K / 128) * (size_t)nvfp4::kPackBlock;
}

int nvfp4_decode_pack(const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, int64_t K, uint8_t *w_packed,
                      void *stream) {
    const char *fn = "nvfp4_decode_pack";
    if (N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 128 != 0) return fail(NVFP4_EUNSUPPORTED, "%s: K (%lld) must be a multiple of 128", fn, (long long)K);
    if (N == 0 || K == 0) return ok();
    if (!w_codes || !w_scales || !w_packed) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (!aligned(w_codes, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 4))
        return fail(NVFP4_EINVAL, "%s: codes and w_packed must be 16-byte, scales 4-byte aligned", fn);
    return hip_status(nvfp4::launch_decode_pack(w_codes, w_scales, N, K, w_packed, as_stream(stream)), "pack kernel");
}

namespace {

// shapes the decode-packed entry points take: 0 <= M <= 64, N >= 0,
// K % 128 == 0, K < 2^24
int check_packed_shape(int64_t M, int64_t N, int64_t K, const char *fn) {
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (M > nvfp4::kSkinnyMaxM)
        return fail(NVFP4_EUNSUPPORTED, "%s: M (%lld) above %lld (decode batches only)", fn, (long long)M,
                    (long long)nvfp4::kSkinnyMaxM);
    if (K % 128 != 0 || K >= nvfp4::kSkinnyMaxK)
        return fail(NVFP4_EUNSUPPORTED, "%s: K (%lld) must be a multiple of 128 below 2^24", fn, (long long)K);
    return NVFP4_OK;
}

int check_packed_w(const uint8_t *w_packed, const float *w_alpha, const char *fn) {
    if (!w_packed || !w_alpha) return fail(NVFP4_EINVAL, "%s: w_packed and w_alpha must be non-null", fn);
    if (!aligned(w_packed, 16)) return fail(NVFP4_EINVAL, "%s: w_packed must be 16-byte aligned", fn);
    return NVFP4_OK;
}

}  // namespace

int nvfp4_gemm_packed(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha, const uint8_t *w_packed,
                      const float *w_alpha, int64_t M, int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "nvfp4_gemm_packed";
    int rc = check_packed_shape(M, N, K, fn);
    if (rc) return rc;
    if (M == 0 || N == 0) return ok();
    if ((rc = check_out(out, out_dtype, N, ld_out, fn))) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if ((rc = check_packed_w(w_packed, w_alpha, fn))) return rc;
    if ((rc = check_nvfp4(a_codes, a_scales, a_alpha, "A", fn))) return rc;
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    return hip_status(nvfp4::launch_skinny_nvfp4(a_codes, a_scales, a_alpha, w_packed, nullptr, w_alpha, M, N, K, out,
                                                 out_dtype, ld_out, workspace, workspace_bytes, s, true),
                      "nvfp4 decode kernel");
}

int nvfp4_quant_gemm_packed(const void *x_bf16, int64_t ld_x, float *a_alpha, int alpha_mode,
                            const uint8_t *w_packed, const float *w_alpha, int64_t M, int64_t N, int64_t K, void *out,
                            int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "nvfp4_quant_gemm_packed";
    int rc = check_packed_shape(M, N, K, fn);
    if (rc) return rc;
    if (alpha_mode != NVFP4_ALPHA_DYNAMIC && alpha_mode != NVFP4_ALPHA_STATIC)
        return fail(NVFP4_EINVAL, "%s: bad alpha_mode %d", fn, alpha_mode);
    if (M == 0 || N == 0) return ok();
    if ((rc = check_out(out, out_dtype, N, ld_out, fn))) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if ((rc = check_packed_w(w_packed, w_alpha, fn))) return rc;
    if (!x_bf16 || !a_alpha) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (ld_x < K || ld_x % 8 != 0) return fail(NVFP4_EINVAL, "%s: ld_x must be >= K and a multiple of 8", fn);
    if (!aligned(x_bf16, 16)) return fail(NVFP4_EINVAL, "%s: x must be 16-byte aligned", fn);
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    const bool dyn = alpha_mode == NVFP4_ALPHA_DYNAMIC;
    if (fused_decode_shape(M, N, K)) {
        if (dyn) {
            const size_t need = (size_t)nvfp4::amax_parts(M, K) * sizeof(uint32_t);
            if (!workspace || workspace_bytes < need)
                return fail(NVFP4_EWORKSPACE, "%s: dynamic alpha needs %zu workspace bytes", fn, need);
        }
        return hip_status(nvfp4::launch_skinny_fused((const uint16_t *)x_bf16, ld_x, a_alpha, dyn, w_packed, nullptr,
                                                     w_alpha, M, N, K, out, out_dtype, ld_out, workspace,
                                                     workspace_bytes, s, true),
                          "fused decode kernel");
    }
    // quantize the batch into the workspace, then the decode kernel
    const QgLayout l = qg_layout(M, N, K, dyn);
    if (!workspace || workspace_bytes < l.split)
        return fail(NVFP4_EWORKSPACE, "%s: needs at least %zu workspace bytes (%zu with the split-K partials)", fn,
                    l.split, l.total);
    uint8_t *wsb = (uint8_t *)workspace;
    uint8_t *codes = wsb + l.codes, *scales = wsb + l.scales;
    const int nparts = nvfp4::amax_parts(M, K);
    if ((rc = hip_status(dyn ? nvfp4::launch_quantize_dynamic((const uint16_t *)x_bf16, M, K, ld_x, codes, scales,
                                                              a_alpha, (uint32_t *)(wsb + l.parts), nparts, s, l.pack_a)
                             : nvfp4::launch_quantize((const uint16_t *)x_bf16, M, K, ld_x, codes, scales, a_alpha, 0,
                                                      nullptr, nparts, s, l.pack_a),
                         "quantize kernel")))
        return rc;
    return hip_status(nvfp4::launch_skinny_nvfp4(codes, scales, a_alpha, w_packed, nullptr, w_alpha, M, N, K, out,
                                                 out_dtype, ld_out, wsb + l.split, workspace_bytes - l.split, s,
                                                 nvfp4::kPackW | (l.pack_a ? nvfp4::kPackA : 0)),
                      "nvfp4 decode kernel");
}

size_t bf16_decode_pack_size(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 32 != 0) return 0;
    return (size_t)((N + 15) / 16) * (size_t)(K / 32) * 1024;
}

int bf16_decode_pack(const void *w_bf16, int64_t N, int64_t K, void *w_packed, void *stream) {
    const char *fn = "bf16_decode_pack";
    if (N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (K % 32 != 0) return fail(NVFP4_EUNSUPPORTED, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
    if (N == 0 || K == 0) return ok();
    if (!w_bf16 || !w_packed) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (!aligned(w_bf16, 16) || !aligned(w_packed, 16))
        return fail(NVFP4_EINVAL, "%s: w and w_packed must be 16-byte aligned", fn);
    return hip_status(nvfp4::launch_bf16_pack((const uint16_t *)w_bf16, N, K, (uint8_t *)w_packed, as_stream(stream)),
                      "pack kernel");
}

int bf16_gemm_packed(const void *a_bf16, const void *w_packed, int64_t M, int64_t N, int64_t K, void *out,
                     int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "bf16_gemm_packed";
    if (M < 0 || N < 0 || K < 0) return fail(NVFP4_EINVAL, "%s: negative size", fn);
    if (M > nvfp4::kSkinnyMaxM)
        return fail(NVFP4_EUNSUPPORTED, "%s: M (%lld) above %lld (decode batches only)", fn, (long long)M,
                    (long long)nvfp4::kSkinnyMaxM);
    if (K % 32 != 0 || K >= nvfp4::kSkinnyMaxK)
        return fail(NVFP4_EUNSUPPORTED, "%s: K (%lld) must be a multiple of 32 below 2^24", fn, (long long)K);
    if (M == 0 || N == 0) return ok();
    int rc = check_out(out, out_dtype, N, ld_out, fn);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const int esz = out_dtype == NVFP4_OUT_F32 ? 4 : 2;
    if (K == 0) return hip_status(nvfp4::launch_fill_zero(out, M, N, ld_out, esz, s), "fill kernel");
    if (!a_bf16 || !w_packed) return fail(NVFP4_EINVAL, "%s: null pointer", fn);
    if (!aligned(a_bf16, 16) || !aligned(w_packed, 16))
        return fail(NVFP4_EINVAL, "%s: a and w_packed must be 16-byte aligned", fn);
    if (workspace && !aligned(workspace, 16)) return fail(NVFP4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    return hip_status(nvfp4::launch_skinny_bf16((const uint16_t *)a_bf16, (const uint16_t *)w_packed, M, N, K, out,
                                                out_dtype, ld_out, workspace, workspace_bytes, s, true),
                      "bf16 decode kernel");
}

}  // extern "C"
