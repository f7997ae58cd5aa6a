/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 prefill GEMM library.
 *
 * Method: "Quantized Prefilling, Precise Decoding for Agentic LLMs"
 * (Mix-Quant), Section 3.3.  Prefill linear layers run as W4A4 GEMMs on
 * NVFP4 tensors; decoding stays in BF16.  An NVFP4 tensor holds E2M1 codes,
 * one FP8 E4M3 scale per 16 consecutive elements along the GEMM reduction
 * dimension K, and one FP32 tensor scale alpha (Eq. 2, Eq. 3).
 *
 * Layouts (row-major, except the decode-packed weights described with
 * nvfp4_decode_pack and bf16_decode_pack; all in device memory owned by the
 * caller):
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

#define NVFP4_ABI_VERSION 3

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
 * Dynamic alpha: an amax pass writes per-workgroup partial maxima to the
 * workspace, then the quantize pass runs; a tensor of at most 65536
 * elements (a decode batch) takes one launch, every workgroup forming the
 * amax itself, and leaves the workspace untouched.
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
 * nvfp4_quantize for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and checks as nvfp4_quantize, without a workspace:
 * in NVFP4_ALPHA_DYNAMIC mode the amax partials live in a scratch array
 * inside the library, 4 KB (1024 partial maxima) per GPU, held by every GPU
 * the library runs on until the process ends.  Every tensor size that
 * nvfp4_quantize accepts fits it (the amax pass never writes more than 1024
 * partials); a larger count would be refused with NVFP4_EUNSUPPORTED.  The
 * call allocates nothing.  All calls on one GPU share that GPU's array and
 * leave their partials in it: calls that overlap on one GPU (on different
 * streams, or from different threads) race and must be ordered by the
 * caller.
 */
int nvfp4_quantize_noalloc(const void *x_bf16, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *codes,
                           uint8_t *scales, float *alpha, int alpha_mode, void *stream);

/* Bytes of device workspace nvfp4_gemm uses at these sizes for its fastest
 * kernels (0: none).  Decode shapes split K over workgroups and keep FP32
 * partial tiles [S][M][N] there. */
size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * NVFP4 x NVFP4 GEMM (the W4A4 prefill linear layer; Mix-Quant Section 3.3
 * and Section 4.2 "Prefilling Stage Speedup"):
 *   Y[m, n] = sum_k xhatA[m, k] * xhatW[n, k],   xhat = alpha * sigma * q (Eq. 2)
 *   a_codes [M, K/2], a_scales [M, K/16], a_alpha float[1]   (activations)
 *   w_codes [N, K/2], w_scales [N, K/16], w_alpha float[1]   (weights)
 *   K % 16 == 0; M, N >= 0; code arrays 16-byte aligned, scale arrays 4-byte aligned
 *   out [M, ld_out] FP32 (NVFP4_OUT_F32) or BF16 (NVFP4_OUT_BF16, nearest-even),
 *   ld_out >= N.  Accumulation is FP32; each product q*sigma is exact.
 *   workspace: NULL, or 16-byte aligned device scratch of workspace_bytes;
 *   contents undefined on entry and exit; a call that overlaps another use of
 *   the same workspace races.  With at least nvfp4_gemm_workspace_size(M, N, K)
 *   bytes the decode kernels split K over workgroups (S slices: partial tiles
 *   summed in slice order by a second kernel); with less they run unsplit.
 * At decode shapes (M <= 64, K % 32 == 0, K < 2^24; the uniform-NVFP4 and
 * FP4-decode variants of Mix-Quant Section 4) the decode kernels stream the
 * weights; otherwise a tile kernel runs.  These kernels, and split and unsplit
 * runs, sum in FP32 but in different orders.
 */
int nvfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
               int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out, void *workspace,
               size_t workspace_bytes, void *stream);

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
 * A dynamic output scale needs the whole output's amax before any block is
 * encoded, so the epilogue cannot apply it: nvfp4_gemm_quant_out_dynamic
 * below forms Y first.
 */
int nvfp4_gemm_quant_out(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                         const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                         int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales, const float *y_alpha,
                         void *stream);

/*
 * nvfp4_gemm_quant_out with a dynamic output tensor scale (Mix-Quant Section
 * 3.3, Eq. 2 and Eq. 3 on the product Y, the tensor scale taken from Y's
 * largest magnitude): alpha_Y = fl32(max |y| / 2688) over every FP32 output
 * y = (acc * alpha_A) * alpha_W (the values nvfp4_gemm's tile kernel gives
 * with an FP32 output), then codes and scales of Y as in
 * nvfp4_gemm_quant_out with that alpha.  The whole Y must be formed before
 * any block is encoded, so the call runs three kernels on the stream: the
 * tile GEMM writing Y in FP32 to the workspace with per-wave maxima of |y|,
 * a one-workgroup reduction to alpha_Y, and an FP32 quantizer.
 *   operands and N, K as in nvfp4_gemm_quant_out
 *   y_alpha float[1] device, written
 *   workspace: 256-byte aligned device scratch of at least
 *   nvfp4_gemm_quant_out_dynamic_workspace_size(M, N, K) bytes (the FP32 Y
 *   and the maxima; contents undefined on entry and exit), else
 *   NVFP4_EWORKSPACE.
 * K == 0 gives alpha_Y = 0 and zero codes and scales.
 */
size_t nvfp4_gemm_quant_out_dynamic_workspace_size(int64_t M, int64_t N, int64_t K);
int nvfp4_gemm_quant_out_dynamic(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                 const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                 int64_t M, int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales,
                                 float *y_alpha, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace nvfp4_quant_gemm uses at these sizes for its
 * fastest path (see nvfp4_quant_gemm). */
size_t nvfp4_quant_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * Prefill linear from BF16 activations: quantization to NVFP4 and the GEMM in
 * one call (Mix-Quant Section 3.3: quantization, dequantization and the
 * matrix product fused by the backend).
 *   x_bf16 [M, ld_x] BF16 (16-byte aligned, ld_x % 8 == 0), K % 16 == 0
 *   a_alpha float[1]: written (dynamic) or read (static) as in nvfp4_quantize
 *   weights, out, out_dtype, ld_out as in nvfp4_gemm
 *   workspace: 16-byte aligned device scratch (contents undefined on entry and
 *   exit); dynamic alpha needs at least nvfp4_quantize_workspace_size(M, K)
 *   bytes (NVFP4_EWORKSPACE otherwise).
 * Paths, by shape and workspace:
 *   - K % 32 == 0 and either M <= 2 with M * K <= 196608, or M <= 6 with
 *     N <= 8192 and M * K <= 32768: one decode kernel quantizes the batch
 *     into LDS in every workgroup (each forms the dynamic alpha itself) and
 *     streams the weights (larger batches, and wider layers, measured faster
 *     quantized once);
 *   - otherwise, with nvfp4_quant_gemm_workspace_size(M, N, K) bytes: the
 *     quantizer writes codes and scales into the workspace and nvfp4_gemm's
 *     kernels run on them (decode batches of 3-64 rows with K % 128 == 0 in
 *     the decode kernel's block layout of nvfp4_decode_pack, so each of its
 *     loads reads 1 KB contiguous; one quantization per activation element; the
 *     in-prologue variant below repeats it for every column tile and measured
 *     slower at every prefill size);
 *   - otherwise: a tile kernel quantizes the activations in its operand
 *     staging (after an amax pass for a dynamic alpha).
 * Results equal nvfp4_quantize followed by nvfp4_gemm (given the workspace
 * sizes of both queries) bit for bit, except between the third path and a
 * decode kernel, or the first path and the tile kernel (M > 64 or
 * K % 32 != 0): there the two sum in different orders (both within FP32
 * rounding of the exact product).
 */
int nvfp4_quant_gemm(const void *x_bf16, int64_t ld_x, float *a_alpha, int alpha_mode,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                     int64_t M, int64_t N, int64_t K, void *out, int out_dtype, int64_t ld_out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode-packed NVFP4 weights for the decode kernels (the uniform-NVFP4
 * decode variant of Mix-Quant Section 4; decode is bound by moving the
 * weights, Section 3.1).  The row-major layout above makes a decode wave's
 * 16-byte loads gather 16 rows per instruction and its block-scale loads
 * scatter; the packed layout stores, for every group of 16 weight rows g and
 * every 128-wide K chunk c, one 1152-byte block at offset
 * (g * K / 128 + c) * 1152:
 *   bytes [0, 1024): byte 16 l + b = code byte 64 c + 16 (l / 16) + b of row
 *                    16 g + l % 16 (l = 0..63, b = 0..15)
 *   bytes [1024, 1152): byte 8 r + t = scale byte 8 c + t of row 16 g + r
 * Rows past N are zeros.  Same codes and scales, so the packed entry points
 * below give the row-major ones' results bit for bit.
 *   nvfp4_decode_pack_size: bytes of the packed weight (0 if N <= 0, K <= 0
 *   or K % 128 != 0).
 *   nvfp4_decode_pack: w_codes [N, K/2] (16-byte aligned), w_scales
 *   [N, K/16] (4-byte aligned) -> w_packed (16-byte aligned, caller-owned,
 *   nvfp4_decode_pack_size bytes).  K % 128 != 0: NVFP4_EUNSUPPORTED.
 */
size_t nvfp4_decode_pack_size(int64_t N, int64_t K);
int nvfp4_decode_pack(const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, int64_t K,
                      uint8_t *w_packed, void *stream);

/*
 * nvfp4_gemm on decode-packed weights: decode batches only (M <= 64; K % 128
 * == 0 and K < 2^24, else NVFP4_EUNSUPPORTED).  Operands other than the
 * weight, out and workspace (nvfp4_gemm_workspace_size(M, N, K) bytes for
 * the split-K partials) as in nvfp4_gemm; results equal nvfp4_gemm's on the
 * row-major weight bit for bit.
 */
int nvfp4_gemm_packed(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                      const uint8_t *w_packed, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                      void *out, int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * nvfp4_quant_gemm on decode-packed weights (M <= 64, K % 128 == 0, K < 2^24,
 * else NVFP4_EUNSUPPORTED): the fused decode kernel for the batches
 * nvfp4_quant_gemm routes to it, otherwise the quantizer into the workspace
 * and the decode kernel.  workspace: nvfp4_quant_gemm_workspace_size(M, N, K)
 * bytes; the fused batches need only what nvfp4_quant_gemm needs for them,
 * the others at least the quantized batch (codes, scales, amax partials),
 * else NVFP4_EWORKSPACE.  Results equal nvfp4_quant_gemm's on the row-major
 * weight bit for bit.
 */
int nvfp4_quant_gemm_packed(const void *x_bf16, int64_t ld_x, float *a_alpha, int alpha_mode,
                            const uint8_t *w_packed, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                            void *out, int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Bytes of device workspace bf16_gemm uses at these sizes for its fastest
 * kernels (0: none); as nvfp4_gemm_workspace_size. */
size_t bf16_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * BF16 GEMM of the high-precision decode path and the prefill baseline
 * (Mix-Quant Section 3.3 "Prefill-Decode Disaggregation Deployment": the
 * decode path keeps the original BF16 model; Section 4.2: the BF16 baseline).
 *   Y[M, N] = A[M, K] * W[N, K]^T, FP32 accumulation
 *   a_bf16 [M, K] and w_bf16 [N, K] contiguous, 16-byte aligned, K % 8 == 0
 *   out [M, ld_out] FP32 or BF16.  Small M (decode batches, M <= 64) uses a
 *   bandwidth-oriented kernel, split over K with a large enough workspace
 *   (as in nvfp4_gemm); large M the MFMA tile kernel.
 */
int bf16_gemm(const void *a_bf16, const void *w_bf16, int64_t M, int64_t N, int64_t K, void *out,
              int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * BF16 decode on decode-packed weights (the decode path of Mix-Quant Section
 * 3.3 keeps the BF16 weights; decode is bound by moving them, Section 3.1).
 * The same BF16 values re-laid out once, so that each 16-byte load of a
 * decode wave reads contiguous memory: for every group of 16 weight rows g
 * and 32-wide K step t, 1 KB at offset (g * K / 32 + t) * 1024 whose byte
 * 16 l + b (l = 0..63, b = 0..15) is byte 16 (l / 16) + b of the 64 bytes of
 * step t in row 16 g + l % 16; rows past N are zeros.
 *   bf16_decode_pack_size: bytes of the packed weight (0 if N <= 0, K <= 0 or
 *   K % 32 != 0).
 *   bf16_decode_pack: w_bf16 [N, K] contiguous (16-byte aligned) -> w_packed
 *   (16-byte aligned, caller-owned).  K % 32 != 0: NVFP4_EUNSUPPORTED.
 *   bf16_gemm_packed: bf16_gemm for decode batches (M <= 64; K % 32 == 0,
 *   K < 2^24, else NVFP4_EUNSUPPORTED) on the packed weight; other arguments
 *   and the workspace (bf16_gemm_workspace_size) as in bf16_gemm.  Results
 *   equal bf16_gemm's on the row-major weight bit for bit.
 */
size_t bf16_decode_pack_size(int64_t N, int64_t K);
int bf16_decode_pack(const void *w_bf16, int64_t N, int64_t K, void *w_packed, void *stream);
int bf16_gemm_packed(const void *a_bf16, const void *w_packed, int64_t M, int64_t N, int64_t K, void *out,
                     int out_dtype, int64_t ld_out, void *workspace, size_t workspace_bytes, void *stream);

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
