/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 prefill GEMM library.
 *
 * Method: "Quantized Prefilling, Precise Decoding for Agentic LLMs"
 * (Mix-Quant), Section 3.3.  Prefill linear layers run as W4A4 GEMMs on
 * NVFP4 tensors; decoding stays in BF16.  An NVFP4 tensor holds E2M1 codes,
 * one FP8 E4M3 scale per 16 consecutive elements along the GEMM reduction
 * dimension K, and one FP32 tensor scale alpha (Eq. 2, Eq. 3).
 *
 * Layouts (all row-major, all in device memory owned by the caller):
 *   BF16 matrix X [rows, cols], row stride ld (elements, >= cols)
 *   codes  uint8 [rows, cols/2]   two E2M1 codes per byte, even element in
 *                                  the low nibble, sign in bit 3 of a nibble
 *   scales uint8 [rows, cols/16]  E4M3 ("FN": bias 7, max 448) block scales
 *   alpha  float [1]               tensor scale, in device memory
 *   GEMM:  Y[M, N] = A[M, K] * W[N, K]^T  (W is a PyTorch Linear weight)
 *
 * Arithmetic of the quantizer, fixed so that codes are bit-exact:
 *   alpha   = fl32(amax(|X|) / 2688)                  (dynamic mode)
 *   s_b     = fl32(amax_b / fl32(alpha * 6))           Eq. 3, 0 if alpha*6 == 0
 *   sigma_b = E4M3 nearest-even of s_b, saturating at 448
 *   q_i     = E2M1 nearest-even of fl32(x_i / fl32(alpha * sigma_b)),
 *             clipped to +-6, sign kept; signed zero when alpha*sigma_b == 0
 *
 * Execution model: every call is asynchronous on the given HIP stream
 * (a hipStream_t passed as void*; NULL is the default stream), allocates
 * no device memory, and does not synchronize.  Pointers must be device
 * pointers (or host pointers the GPU can read, for alpha in static mode).
 * Arguments are checked before any launch; asynchronous device faults show
 * at the caller's next synchronization.  Inputs must be finite.
 *
 * Errors: 0 on success, otherwise a negative NVFP4_E* status;
 * nvfp4_last_error() returns a thread-local message for the last failure.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

enum {
    NVFP4_OK = 0,
    NVFP4_EINVAL = -1,       /* null pointer, bad size, stride, alignment or dtype */
    NVFP4_EUNSUPPORTED = -2, /* a shape or mode the kernels do not cover            */
    NVFP4_EHIP = -3,         /* a HIP launch or runtime call failed                 */
    NVFP4_EWORKSPACE = -4    /* workspace missing or smaller than required          */
};

enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 };
enum { NVFP4_ALPHA_DYNAMIC = 0, NVFP4_ALPHA_STATIC = 1 };

/* ABI version of the loaded library (NVFP4_ABI_VERSION). */
int nvfp4_abi_version(void);

/* Message for the last failed call on this thread ("" if none). */
const char *nvfp4_last_error(void);

/* Bytes of device workspace nvfp4_quantize needs for a rows x cols tensor in
 * dynamic-alpha mode (0 is enough in static mode).  The workspace holds
 * per-workgroup partial maxima; its contents need no initialisation and are
 * garbage after the call. */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);

/*
 * BF16 -> NVFP4 quantization (Mix-Quant Section 3.3, Eq. 3 then Eq. 2).
 *   x_bf16   [rows, ld_x] BF16, 16-byte aligned, ld_x % 8 == 0
 *   rows>=0, cols >= 0 with cols % 16 == 0 (one block is 16 elements)
 *   codes    [rows, cols/2] uint8 out, 16-byte aligned
 *   scales   [rows, cols/16] uint8 out
 *   alpha    float[1]: written in NVFP4_ALPHA_DYNAMIC mode, read in
 *            NVFP4_ALPHA_STATIC mode (a tensor scale fixed ahead of time)
 *   workspace/workspace_bytes: see nvfp4_quantize_workspace_size
 * rows == 0 or cols == 0: nothing is launched (dynamic alpha is not written).
 * cols >= 2^30 or rows * ceil(cols / 2048) >= 2^31: NVFP4_EUNSUPPORTED (the
 * kernels index a row and the work items with 32-bit offsets).
 */
int nvfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                   uint8_t *scales, float *alpha, int alpha_mode, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * NVFP4 x NVFP4 GEMM (the W4A4 prefill linear layer; Mix-Quant Section 3.3
 * and Section 4.2 "Prefilling Stage Speedup"):
 *   Y[m, n] = sum_k xhatA[m, k] * xhatW[n, k],   xhat = alpha * sigma * q (Eq. 2)
 *   a_codes [M, K/2], a_scales [M, K/16], a_alpha float[1]   (activations)
 *   w_codes [N, K/2], w_scales [N, K/16], w_alpha float[1]   (weights)
 *   K % 16 == 0; M, N >= 0; code arrays 16-byte aligned, scale arrays 4-byte aligned
 *   out [M, ld_out] FP32 (NVFP4_OUT_F32) or BF16 (NVFP4_OUT_BF16, nearest-even),
 *   ld_out >= N.  Accumulation is FP32; each product q*sigma is exact.
 * At decode shapes (M <= 64, K % 32 == 0, K < 2^24; the uniform-NVFP4 and FP4-decode
 * variants of Mix-Quant Section 4) a split-K kernel streams the weights;
 * otherwise a tile kernel runs.  Both sum in FP32 but in different orders.
 */
int nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
               int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out, void *stream);

/*
 * NVFP4 x NVFP4 GEMM whose output is itself NVFP4, for the next linear layer
 * (Mix-Quant Section 3.3: the backend fuses quantization into the matrix
 * product).  Y = xhatA * xhatW^T is formed as nvfp4_gemm's FP32 output
 * (y = (acc * alpha_A) * alpha_W) and quantized in the epilogue with Eq. 3
 * and Eq. 2 against a static output tensor scale:
 *   y_codes [M, N/2] uint8 out (4-byte aligned), y_scales [M, N/16] uint8 out,
 *   y_alpha float[1] in (device): the output tensor scale, e.g. calibrated.
 *   N % 16 == 0, K % 16 == 0; operands as in nvfp4_gemm.  The codes equal
 *   those the quantizer gives for the FP32 output of the same product.
 * A dynamic output scale would need the whole output's amax before any
 * block is quantized, so it is not offered here.
 */
int nvfp4_gemm_quant_out(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                         const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                         int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales, const float *y_alpha,
                         void *stream);

/* Bytes of device workspace nvfp4_quant_gemm needs (dynamic-alpha mode). */
size_t nvfp4_quant_gemm_workspace_size(int64_t M, int64_t K);

/*
 * Fused prefill linear: BF16 activations are quantized to NVFP4 inside the
 * GEMM's operand staging (Mix-Quant Section 3.3: quantization, dequantization
 * and the matrix product fused by the backend).  No codes or scales are
 * written.  For M <= 16 with M * K <= 196608 and K % 32 == 0 a decode kernel
 * quantizes the batch into LDS (every workgroup forms the dynamic alpha
 * itself); otherwise an amax pass precedes a tile kernel that quantizes in its
 * operand staging.  The result equals nvfp4_quantize followed by nvfp4_gemm
 * bit for bit whenever both run decode kernels (the condition above) or both
 * run tile kernels (M > 64 or K % 32 != 0); in between they sum in different
 * orders (both within FP32 rounding of the exact product).
 *   x_bf16 [M, ld_x] BF16 (16-byte aligned, ld_x % 8 == 0), K % 16 == 0
 *   a_alpha float[1]: written (dynamic) or read (static) as in nvfp4_quantize
 *   weights, out, out_dtype, ld_out as in nvfp4_gemm
 */
int nvfp4_quant_gemm(const void *x_bf16, int64_t ld_x, float *a_alpha, int alpha_mode,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                     int64_t M, int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * BF16 GEMM of the high-precision decode path and the prefill baseline
 * (Mix-Quant Section 3.3 "Prefill-Decode Disaggregation Deployment": the
 * decode path keeps the original BF16 model; Section 4.2: the BF16 baseline).
 *   Y[M, N] = A[M, K] * W[N, K]^T, FP32 accumulation
 *   a_bf16 [M, K] and w_bf16 [N, K] contiguous, 16-byte aligned, K % 8 == 0
 *   out [M, ld_out] FP32 or BF16.  Small M (decode batches) uses a
 *   bandwidth-oriented kernel; large M the MFMA tile kernel.
 */
int bf16_gemm(const void *a_bf16, const void *w_bf16, int64_t M, int64_t N, int64_t K, void *out,
              int out_dtype, int64_t ld_out, void *stream);

/*
 * MXFP4 (Mix-Quant Section 3.3 names it as the coarser microscaling format
 * with larger groups and power-of-two scales): E2M1 codes as above and one
 * E8M0 scale byte (value 2^(code - 127)) per 32 consecutive elements, no
 * tensor scale.  Rounding follows the OCP MX v1.0 conversion: shared
 * exponent floor(log2(max |x|)) - 2 clamped to [-127, 127] (-127 for an
 * all-zero block), elements x / 2^shared to E2M1 nearest-even, saturating.
 *   x_bf16 [rows, ld_x] BF16 (16-byte aligned, ld_x % 8 == 0), cols % 32 == 0
 *   codes  [rows, cols/2] uint8 out (16-byte aligned)
 *   scales [rows, cols/32] uint8 out (E8M0)
 */
int mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                   uint8_t *scales, void *stream);

/*
 * MXFP4 x MXFP4 GEMM on gfx950's block-scaled FP4 MFMAs:
 *   Y[m, n] = sum_b 2^(sA[m,b] + sW[n,b]) sum_{k in b} qA[m,k] qW[n,k]
 *   a_codes [M, K/2], a_scales [M, K/32], w_codes [N, K/2], w_scales [N, K/32]
 *   K % 32 == 0; code arrays 16-byte aligned, scale arrays 8-byte aligned
 *   out [M, ld_out] FP32 or BF16 (nearest-even), FP32 accumulation.
 */
int mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
               const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *out, int out_dtype,
               int64_t ld_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
