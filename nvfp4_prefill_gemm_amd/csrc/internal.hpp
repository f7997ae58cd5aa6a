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

// Small tensors (rows * cols <= kSelfAmaxMaxElems, e.g. decode batches) take
// a single launch in dynamic mode: every workgroup of the quantize pass reads
// the whole tensor for its amax, and no amax pass (nor its partials) is used.
// Two rounds of 16 loads per thread (65536 elements) measured faster than the
// two launches (Qwen3-8B decode step at batch 16: 65.0 -> 61.0 us), three or
// four rounds slower (batch 32: 78.9 -> 82.0 us).
constexpr int64_t kSelfAmaxMaxElems = int64_t(1) << 16;
bool quantize_self_amax(int64_t rows, int64_t cols);

// dynamic != 0: alpha = amax / 2688 is written to *alpha, the amax taken from
// partials[0..nparts), or from the tensor itself when quantize_self_amax().
// pack_a: codes and scales go to `codes` in the decode kernel's packed block
// layout (decode_pack_a_bytes(rows, cols) bytes, cols % 128 == 0; rows of the
// last group past `rows` are left unwritten; `scales` unused).
hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint8_t *scales, float *alpha, int dynamic, const uint32_t *partials,
                           int nparts, hipStream_t s, bool pack_a = false);

// Dynamic-alpha quantization: the single launch of quantize_self_amax()
// tensors, else the amax pass into partials (amax_parts(rows, cols) = nparts
// entries) and the quantize pass.
hipError_t launch_quantize_dynamic(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                                   uint8_t *scales, float *alpha, uint32_t *partials, int nparts, hipStream_t s,
                                   bool pack_a = false);

// Device address and size of this device's scratch array for the amax
// partials of nvfp4_quantize_noalloc (looked up once per device).
hipError_t quantize_scratch(uint32_t **ptr, size_t *bytes);

// alpha from partials only (fused path, dynamic mode).
hipError_t launch_alpha_from_partials(const uint32_t *partials, int nparts, float *alpha, hipStream_t s);

// OUT_F32_AMAX: FP32 output plus, per workgroup, eight slots of the waves'
// max |y| (FP32 bits; unused slots 0) for a dynamic output tensor scale.
enum OutType { OUT_F32 = 0, OUT_BF16 = 1, OUT_NVFP4 = 2, OUT_F32_AMAX = 3 };

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

// Tile GEMM with FP32 output y [M, N] (row stride N) and the per-wave maxima
// of |y| in `parts` (gemm_amax_parts(M, N) slots).
hipError_t launch_gemm_nvfp4_f32_amax(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                      const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                      int64_t M, int64_t N, int64_t K, float *y, uint32_t *parts, hipStream_t s);
// Slots launch_gemm_nvfp4_f32_amax writes for this shape (8 per output
// tile), and an upper bound over every tile choice.
int64_t gemm_amax_parts(int64_t M, int64_t N);
int64_t gemm_amax_parts_bound(int64_t M, int64_t N);

// Eq. 3 / Eq. 2 on an FP32 tensor y [rows, ld] (cols % 16 == 0) with the
// tensor scale *alpha (device pointer): codes [rows, cols/2] (4-byte
// aligned), scales [rows, cols/16].
hipError_t launch_quantize_f32(const float *y, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                               uint8_t *scales, const float *alpha, hipStream_t s);

hipError_t launch_gemm_fused(const uint16_t *x, int64_t ld_x, const float *a_alpha,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                             int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                             hipStream_t s);

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                            void *out, int out_type, int64_t ld_out, hipStream_t s);

// Decode kernels (M <= kSkinnyMaxM): a workgroup owns ng 16-column groups and
// one of s K slices; s > 1 writes FP32 partials [s][M][N] to a workspace and
// a reduction kernel sums them in slice order.
enum DecodeKind { DECODE_BF16 = 0, DECODE_NVFP4 = 1, DECODE_FUSED = 2 };
struct DecodePlan {
    int ng, waves, u, s;  // 16-column groups per workgroup, waves, K steps per stage, K slices
    bool pipe = true;     // K loop with each stage's loads pinned ahead of the other's MFMAs
};
DecodePlan decode_plan(int kind, int64_t M, int64_t N, int64_t K);
// NVFP4 decode of one or two batch rows with K % 128 == 0 runs the weight
// codes through the FP4 MFMA (block partial sums scaled afterwards).
inline bool decode_fp4_form(int64_t M, int64_t K) { return M <= 2 && (K & 127) == 0; }
// Workspace bytes of the plan's split-K partials (0 without a split).
size_t decode_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K);

// ws / ws_bytes: the split-K partials; a workspace smaller than
// decode_workspace_bytes() runs the plan without a split.  packed: w is the
// BF16 decode-packed weight (K % 32 == 0): for 16-row group g and 32-wide K
// step t, 1 KB at (g * K / 32 + t) * 1024 whose byte 16 l + b is byte
// 16 (l / 16) + b of row 16 g + l % 16's step t (64 bytes); rows past N zero.
hipError_t launch_skinny_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                              int out_type, int64_t ld_out, void *ws, size_t ws_bytes, hipStream_t s,
                              bool packed = false);
hipError_t launch_bf16_pack(const uint16_t *w, int64_t N, int64_t K, uint8_t *w_packed, hipStream_t s);

// Decode-packed NVFP4 weights (nvfp4_decode_pack): for every group of 16
// rows g and 128-wide K chunk c, one block of kPackBlock bytes at
// (g * K / 128 + c) * kPackBlock: 1024 code bytes, byte 16 l + b = code byte
// 64 c + 16 (l / 16) + b of row 16 g + l % 16 (the 16 bytes lane l of a
// decode wave loads), then 128 scale bytes, byte 8 r + t = scale 8 c + t of
// row 16 g + r.  Rows past N are zeros.  Needs K % 128 == 0.
constexpr int64_t kPackBlock = 1152;
hipError_t launch_decode_pack(const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, int64_t K,
                              uint8_t *w_packed, hipStream_t s);

// NVFP4 x NVFP4 at decode shapes: M <= kSkinnyMaxM, K % 32 == 0, codes
// 16-byte and scales 2-byte aligned (nvfp4_gemm checks and otherwise uses the
// tile kernel).  packed: kPackW, w_codes is the decode-packed weight
// (w_scales unused, K % 128 == 0); kPackA, a_codes holds the activation in
// the same block layout (a_scales unused; K % 128 == 0 and not the FP4-MFMA
// form, i.e. M > 2), as launch_quantize writes it with pack_a.
constexpr int kPackW = 1, kPackA = 2;
hipError_t launch_skinny_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                               int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, void *ws,
                               size_t ws_bytes, hipStream_t s, int packed = 0);
// Activation batches that nvfp4_quant_gemm quantizes into its workspace in
// the packed block layout for the decode kernel.
inline bool decode_pack_a_route(int64_t M, int64_t K) { return M > 2 && M <= 64 && K % 128 == 0; }
// Bytes of an [M, K] activation in that layout: one kPackBlock block per 16
// rows (the last group padded) and 128-wide chunk.
inline size_t decode_pack_a_bytes(int64_t M, int64_t K) {
    return (size_t)((M + 15) / 16) * (size_t)(K / 128) * (size_t)kPackBlock;
}

// Fused decode (BF16 activations quantized into LDS by every workgroup):
// M <= 16, M * K <= kFusedDecodeMaxElems, K % 32 == 0, x rows 16-byte
// aligned; dynamic != 0 computes alpha_A in every workgroup; packed as above.
hipError_t launch_skinny_fused(const uint16_t *x, int64_t ld_x, float *a_alpha, int dynamic,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                               int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, void *ws,
                               size_t ws_bytes, hipStream_t s, bool packed = false);

// nvfp4_quant_gemm routes to the fused decode kernel batches of at most
// kFusedDecodeMaxM rows with M * K <= kFusedDecodeMaxElems (108 KB of codes
// and scales in LDS: every Qwen3-8B layer at 16 tokens), and batches of at
// most kFusedDecodeWideM rows on layers of at most kFusedDecodeWideN
// columns whose batch fits a workgroup's registers (M * K <=
// kFusedDecodeRegElems): there the per-workgroup quantization costs less
// than a separate quantizer launch (measured at batch 3-6 on the Qwen3-8B
// qkv and o projections; at batch 8 quantizing once into the packed block
// layout is faster), while wide layers repeat it too often.
constexpr int64_t kFusedDecodeMaxM = 2;
constexpr int64_t kFusedDecodeMaxElems = 16 * 12288;
constexpr int64_t kFusedDecodeWideM = 6;
constexpr int64_t kFusedDecodeWideN = 8192;
constexpr int64_t kFusedDecodeRegElems = 32768;
inline bool fused_decode_route(int64_t M, int64_t N, int64_t K) {
    if (K % 32 != 0 || M * K > kFusedDecodeMaxElems) return false;
    return M <= kFusedDecodeMaxM || (M <= kFusedDecodeWideM && N <= kFusedDecodeWideN && M * K <= kFusedDecodeRegElems);
}

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
