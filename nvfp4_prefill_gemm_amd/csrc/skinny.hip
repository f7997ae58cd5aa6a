// Decode-shape GEMMs for small batches (M <= 64): Y[M, N] = X[M, K] * W[N, K]^T.
//
// BF16: decode keeps the original BF16 weights (Mix-Quant Section 3.3,
// "Prefill-Decode Disaggregation Deployment") and is bound by streaming W
// from HBM: 2*N*K bytes against 2*M*N*K flops.  A workgroup owns a strip of
// NG*16 weight rows and one slice of K (grid: column strips x K slices); its
// waves split the slice in 32-wide steps (interleaved, so the waves of a
// workgroup read neighbouring 64-byte pieces of the same rows), load through
// buffer resources over the valid rows (steps past the slice or K and rows
// past N or M read zeros, so the loop has no branches), keep two register
// stages of U steps in flight, and run 16x16x32 BF16 MFMAs with X
// zero-padded to MG*16 rows.  The per-wave partial tiles are summed through
// LDS at the end.
//
// Splitting K over workgroups: without it every workgroup of a narrow strip
// streams the whole batch X, so at batch 32-64 the batch bytes crossing L2
// exceed the weight bytes several times over.  With S slices a strip of
// S times as many columns keeps the same number of workgroups, and each reads
// only its slice of X.  Each workgroup then writes its FP32 partial tile to a
// caller-provided workspace [S][M][N], and a second kernel sums the S
// partials in slice order (deterministic) and applies the epilogue.
//
// NVFP4 (both operands E2M1 + E4M3 per 16, the uniform-NVFP4 and
// FP4-decode variants of Mix-Quant's ablations, Section 4): the same layout
// streams 0.5625 bytes per weight instead of 2.  A lane's 16-byte code
// load covers 32 consecutive K; the four 16x16x32 MFMA sub-steps of a
// 128-wide K chunk take its four 8-code words, so sub-step t of lane group g
// holds K = 128c + 32g + 8t + i on both operands (the same permutation of K
// for A and W, which leaves the dot product unchanged).  Codes are expanded
// exactly to q * sigma in FP16 in registers; alpha_A * alpha_W is applied in
// the epilogue as in the prefill GEMM.  Batches of one or two rows with
// K % 128 == 0 skip the expansion: the same 16-byte code loads feed the FP4
// MFMA, whose spare rows separate the 16-element blocks, and each block's
// exact partial sum is scaled by sigma_A * sigma_W in FP32 (see kF4 below).
//
// Fused decode (nvfp4_quant_gemm with M * K <= 196608): the workgroup first
// quantizes the part of the BF16 batch its K slice needs, one 8-element group
// per thread with the quantizer's own Eq. 3 / Eq. 2 functions, into LDS (a
// dynamic tensor scale is formed from a first pass over the whole batch;
// every workgroup derives the same alpha_A and workgroup 0 stores it), then
// runs the loop above with the activation codes read from LDS.  Codes, scales
// and the summation order equal those of quantize followed by the decode GEMM
// with the same slicing, so the two paths agree bit for bit.
//
// Weight layouts: row-major as above, or decode-packed (made once by the
// pack kernels below): each 16-row group's K chunk (128 wide for NVFP4, with
// its scales; 32 wide for BF16) stored as one contiguous block in the order
// the decode lanes load it, so each 16-byte-per-lane load instruction reads
// 1 KB of consecutive bytes instead of 64 bytes from each of 16 rows.  Only
// the weight offsets differ (a per-chunk stride), so both layouts give the
// same results bit for bit.  The NVFP4 activation of more than two rows can
// come in the same block layout (16 batch rows per block, written so by the
// quantizer for nvfp4_quant_gemm's quantize-first decode batches): the batch,
// which every workgroup re-reads in full, then also moves 1 KB contiguous
// per load instruction.
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(4))) float f4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

__device__ __forceinline__ uint2 buf_load8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Epilogue of a decode workgroup: the final output (FP32 or BF16, y =
// (sum * sa) * sw), or the raw FP32 partial of K slice blockIdx.y into the
// workspace [S][M][N].
enum DecOut { DOUT_F32 = 0, DOUT_BF16 = 1, DOUT_PARTIAL = 2 };

// Sum the per-wave 16x16 partial tiles of a workgroup through LDS, one
// (row group, column group) tile at a time, and store them:
// out[m = i*16 + (l>>4)*4 + r][n = n0 + j*16 + (l & 15)].
template <int MG, int NG, int WAVES, int kOut>
__device__ __forceinline__ void tile_reduce(const f4_t (&acc)[MG][NG], float sa, float sw, int64_t M, int64_t N,
                                            int64_t n0, void *__restrict__ out, int64_t ld_out) {
    __shared__ float red[WAVES][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (i + j > 0) __syncthreads();  // previous tile consumed
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][lane][r] = acc[i][j][r];
            __syncthreads();
            for (int idx = threadIdx.x; idx < 256; idx += WAVES * 64) {
                const int r = idx & 3, l = idx >> 2;
                float s = 0.f;
#pragma unroll
                for (int v = 0; v < WAVES; ++v) s += red[v][l][r];
                const int64_t m = i * 16 + (l >> 4) * 4 + r, n = n0 + j * 16 + (l & 15);
                if (m < M && n < N) {
                    if constexpr (kOut == DOUT_PARTIAL) {
                        reinterpret_cast<float *>(out)[((int64_t)blockIdx.y * M + m) * N + n] = s;
                    } else {
                        const float y = (s * sa) * sw;
                        if constexpr (kOut == DOUT_BF16)
                            reinterpret_cast<uint16_t *>(out)[m * ld_out + n] = (uint16_t)f32_to_bf16_bits(y);
                        else
                            reinterpret_cast<float *>(out)[m * ld_out + n] = y;
                    }
                }
            }
        }
}

// K steps [sb, se) of this workgroup's slice: slice blockIdx.y of `sps` steps.
__device__ __forceinline__ void slice_steps(int64_t steps, int64_t sps, int64_t &sb, int64_t &se) {
    sb = (int64_t)blockIdx.y * sps;
    se = sb + sps < steps ? sb + sps : steps;
}

template <int MG, int NG, int WAVES, int U, int kOut, bool kPipe>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                            int64_t M, int64_t N, int64_t K, void *__restrict__ out,
                                                            int64_t ld_out, int64_t sps, int packed) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * (NG * 16);
    const int kq = (lane >> 4) * 8;
    int64_t sb, se;
    slice_steps((K + 31) >> 5, sps, sb, se);

    f4_t acc[MG][NG];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    // buffer resources over this workgroup's weight rows and over X: rows past
    // N or M and steps past the slice or K read zeros (offset beyond the
    // resource).  A lane's weight bytes of step ks are at wro + ks * wstep:
    // row-major W [N, K] (step 64), or the decode-packed blocks (1 KB per 16
    // rows and step, in lane order; step 1 KB; K % 32 == 0).
    const int64_t nrows = N - n0 < NG * 16 ? N - n0 : NG * 16;
    const int64_t gbytes = (K >> 5) * 1024, ngroups = (nrows + 15) >> 4;  // packed bytes per 16-row group
    const rsrc_t wrs = packed ? make_rsrc(w + (n0 >> 4) * (gbytes >> 1), (uint32_t)(ngroups * gbytes))
                              : make_rsrc(w + n0 * K, (uint32_t)(nrows * K * 2));
    const uint32_t wstep = packed ? 1024u : 64u;
    const rsrc_t xrs = make_rsrc(x, (uint32_t)(M * K * 2));
    uint32_t wro[NG], xro[MG];  // byte offsets of this lane's rows
#pragma unroll
    for (int j = 0; j < NG; ++j)
        wro[j] = packed ? (uint32_t)(j * gbytes + lane * 16) : (uint32_t)((j * 16 + (lane & 15)) * K * 2 + kq * 2);
#pragma unroll
    for (int i = 0; i < MG; ++i) xro[i] = (uint32_t)((i * 16 + (lane & 15)) * K * 2);

    // Two register stages of U K-steps each: the loads of the next stage are
    // issued before the MFMAs of the current one, so every wave keeps loads in
    // flight while it computes.
    typedef uint4 WStage[U][NG];
    typedef uint4 XStage[U][MG];
    auto load = [&](int64_t ks0, WStage &bw, XStage &ax) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t ks = ks0 + (int64_t)u * WAVES, k = ks * 32 + kq;
            const bool kin = ks < se && k + 8 <= K;
#pragma unroll
            for (int j = 0; j < NG; ++j) bw[u][j] = buf_load16(wrs, kin ? wro[j] + (uint32_t)ks * wstep : kBufOOB);
#pragma unroll
            for (int i = 0; i < MG; ++i) ax[u][i] = buf_load16(xrs, kin ? xro[i] + (uint32_t)(k * 2) : kBufOOB);
        }
    };
    auto compute = [&](const WStage &bw, const XStage &ax) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < MG; ++i)
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[u][i]),
                                                                        __builtin_bit_cast(bf16x8_t, bw[u][j]),
                                                                        acc[i][j], 0, 0, 0);
    };
    const int64_t stride = (int64_t)WAVES * U;
    WStage bw0, bw1;
    XStage ax0, ax1;
    int64_t k = sb + wave;
    load(k, bw0, ax0);
    if constexpr (kPipe) {
        // Two steps per trip with no exit test between a stage's loads and
        // its MFMAs: given one, the compiler sinks the loads past it to their
        // use and then waits for every load before each step.  The
        // scheduling barriers keep each stage's loads ahead of the other
        // stage's MFMAs, so one stage is always in flight.  A step past the
        // slice reads zeros (at most one per wave; its MFMAs add nothing).
        for (;;) {
            load(k + stride, bw1, ax1);
            __builtin_amdgcn_sched_barrier(0);
            compute(bw0, ax0);
            load(k + 2 * stride, bw0, ax0);
            __builtin_amdgcn_sched_barrier(0);
            compute(bw1, ax1);
            k += 2 * stride;
            if (k >= se) break;
        }
    } else {
        // the compiler's own schedule: both stages' loads issued together,
        // then both consumed (faster for one column group of 16 waves)
        for (;;) {
            const int64_t k1 = k + stride;
            load(k1, bw1, ax1);
            compute(bw0, ax0);
            if (k1 >= se) break;
            const int64_t k2 = k1 + stride;
            load(k2, bw0, ax0);
            compute(bw1, ax1);
            if (k2 >= se) break;
            k = k2;
        }
    }

    tile_reduce<MG, NG, WAVES, kOut>(acc, 1.0f, 1.0f, M, N, n0, out, ld_out);
}

// Source of the A operand of the NVFP4 decode kernel.
enum ASrc { A_NVFP4 = 0, A_BF16_DYNAMIC = 1, A_BF16_STATIC = 2 };

// NVFP4 x NVFP4, M <= MG*16, NG*16 weight rows per workgroup, K % 32 == 0,
// 16-byte aligned codes and 4-byte aligned scales.  kA != A_NVFP4: A is
// BF16 [M, ld_x] (16-byte aligned rows, MG == 1), quantized into LDS
// (M * K * 9 / 16 bytes of dynamic shared memory; the slice's part is filled).
//
// kF4 (M <= 2, K % 128 == 0, MG == 1): the weight codes go to the FP4 MFMA
// as they are loaded.  One v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0
// scales) per 128-wide chunk and 16 weight rows: A row r holds block r % 8 of
// the chunk for batch row r / 8 and zeros elsewhere, so output element
// (r, n) is that block's partial sum of E2M1 products, exact in FP32 (at most
// 16 products of magnitude <= 36, multiples of 1/4).  It is then scaled by
// sigma_A * sigma_W (exact: two 4-bit significands) and added to the lane's
// FP32 accumulator for that block position, so no code is expanded to FP16.
// A lane holds rows 4 (l / 16) + i, i.e. batch row l / 32 and blocks
// 4 ((l / 16) % 2) + i of every chunk; the four block sums of a lane and the
// two lanes of a batch row are added at the end.
template <int MG, int NG, int WAVES, int U, int kOut, int kA = A_NVFP4, bool kF4 = false, bool kPipe = true>
__global__ __launch_bounds__(WAVES * 64) void skinny_nvfp4_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, float *__restrict__ a_alpha,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, const float *__restrict__ w_alpha, int64_t M,
    int64_t N, int64_t K, void *__restrict__ out, int64_t ld_out, const uint16_t *__restrict__ x, int64_t ld_x,
    int64_t sps, int packed) {
    static_assert(kA == A_NVFP4 || MG == 1, "BF16 activations: one 16-row group");
    static_assert(!kF4 || MG == 1, "the FP4-MFMA path takes at most two batch rows");
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * (NG * 16);
    const int64_t cb = K >> 1, sb = K >> 4;  // code and scale bytes per row
    int64_t cs, ce;                          // this slice's 128-wide K chunks [cs, ce)
    slice_steps((K + 127) >> 7, sps, cs, ce);
    const int kg = (lane >> 4) * 32;         // this lane group's K offset in a chunk

    f4_t acc[MG][NG];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    // buffer resources over this workgroup's weight rows (and over A in global
    // memory): rows past N or M and chunks past the slice or K read zeros.
    // Weight offsets are this lane's bytes of chunk 0 plus chunk * wstep:
    // row-major codes [N, K/2] and scales [N, K/16] (steps 64 and 8), or the
    // decode-packed blocks (one 1152-byte block per 16 rows and chunk, both
    // steps 1152; rows past N are zeros in the last group's blocks).
    // The activation codes may come in the same packed layout (kPackA: made
    // by the quantizer for nvfp4_quant_gemm's quantize-first batches, A_NVFP4
    // without the FP4-MFMA form): then a row group's chunk is one block too.
    const bool wpk = packed & kPackW, apk = packed & kPackA;
    const int64_t nrows = N - n0 < NG * 16 ? N - n0 : NG * 16;
    const int64_t nchunks = K >> 7, gbytes = nchunks * kPackBlock;  // packed bytes per 16-row group
    const int64_t ngroups = (nrows + 15) >> 4;
    const rsrc_t wcs = wpk ? make_rsrc(wc + (n0 >> 4) * gbytes, (uint32_t)(ngroups * gbytes))
                           : make_rsrc(wc + n0 * cb, (uint32_t)(nrows * cb));
    const rsrc_t wss = wpk ? wcs : make_rsrc(ws + n0 * sb, (uint32_t)(nrows * sb));
    const uint32_t cstep = wpk ? (uint32_t)kPackBlock : 64u, sstep = wpk ? (uint32_t)kPackBlock : 8u;
    const rsrc_t xcs = apk ? make_rsrc(ac, (uint32_t)(((M + 15) >> 4) * gbytes)) : make_rsrc(ac, (uint32_t)(M * cb));
    const rsrc_t xss = apk ? xcs : make_rsrc(as, (uint32_t)(M * sb));
    uint32_t wco[NG], wso[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int r = j * 16 + (lane & 15);
        wco[j] = wpk ? (uint32_t)(j * gbytes + lane * 16) : (uint32_t)(r * cb + (lane >> 4) * 16);
        wso[j] = wpk ? (uint32_t)(j * gbytes + 1024 + (lane & 15) * 8 + (lane >> 4) * 2)
                     : (uint32_t)(r * sb + (lane >> 4) * 2);
    }
    // A offsets of chunk 0 (row-major: the row's start; the lane's K part
    // and the chunk are added per load) and, packed, the lane's bytes of
    // chunk 0 in its row group's blocks (+ kPackBlock per chunk)
    uint32_t xco[MG], xso[MG], xpo[MG];
    bool xv[MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) {
        const int64_t m = i * 16 + (lane & 15);
        xv[i] = m < M;
        xco[i] = (uint32_t)((xv[i] ? m : 0) * cb);
        xso[i] = (uint32_t)((xv[i] ? m : 0) * sb);
        xpo[i] = (uint32_t)(i * gbytes + lane * 16);
    }
    const uint32_t xps = 1024u + (uint32_t)((lane & 15) * 8 + (lane >> 4) * 2) - (uint32_t)(lane * 16);  // code -> scale
    // kF4: this lane's A-operand piece (8 code bytes of block fr % 8 of batch
    // row fr / 8, in half fr % 2 of the lane's 32 K, when that block lies in
    // the lane's K range) and its output rows' scale words (4 bytes: blocks
    // 4 (fg % 2) .. + 3 of the chunk, for batch row lane / 32 and weight row n)
    const int fr = lane & 15, fg = lane >> 4;
    const bool f_act = ((fr & 7) >> 1) == fg && (fr >> 3) < M, f_hi = fr & 1;
    const bool f_sact = (lane >> 5) < M;
    const uint32_t f_xo = f_act ? (uint32_t)((fr >> 3) * cb + 8 * (fr & 7)) : 0u;   // + 64 per chunk
    const uint32_t f_so = (uint32_t)((f_sact ? (lane >> 5) : 0) * sb + 4 * (fg & 1));  // + 8 per chunk
    uint32_t f_wso[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j)
        f_wso[j] = wpk ? (uint32_t)(j * gbytes + 1024 + (lane & 15) * 8 + 4 * (fg & 1))
                          : (uint32_t)((j * 16 + (lane & 15)) * sb + 4 * (fg & 1));
    const uint8_t *lc = nullptr, *ls = nullptr;  // LDS copy of A (fused path)
    float alpha_a = 0.0f;
    // Two register stages of U chunks each, as in the BF16 decode kernel.
    struct NStage {
        uint4 wq[U][NG], xq[U][MG];
        uint32_t wsc[U][NG], xsc[U][MG];
        uint2 fx[U];  // kF4
        uint32_t fxs[U], fws[U][NG];
    };
    // weights (w) and the batch (x) of a stage; the fused path issues the
    // first stage's weight loads before it quantizes the batch
    auto load_part = [&](int64_t c0, NStage &st, bool do_w, bool do_x) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * WAVES, k = c * 128 + kg;
            const bool kin = c < ce && k < K;  // K % 32 == 0: the lane's 32 codes are all in or all out
            const uint32_t kc = (uint32_t)(k >> 1), ksc = (uint32_t)(k >> 4);
            if constexpr (kF4) {  // K % 128 == 0: the whole chunk is in range
                if (do_w) {
#pragma unroll
                    for (int j = 0; j < NG; ++j) {
                        st.wq[u][j] = buf_load16(wcs, kin ? wco[j] + (uint32_t)c * cstep : kBufOOB);
                        st.fws[u][j] = buf_load4(wss, kin ? f_wso[j] + (uint32_t)c * sstep : kBufOOB);
                    }
                }
                if (!do_x) continue;
                if constexpr (kA == A_NVFP4) {
                    st.fx[u] = buf_load8(xcs, (kin & f_act) ? f_xo + (uint32_t)c * 64u : kBufOOB);
                    st.fxs[u] = buf_load4(xss, (kin & f_sact) ? f_so + (uint32_t)c * 8u : kBufOOB);
                } else {  // LDS: clamp the address, zero by select
                    const uint32_t cc = kin ? (uint32_t)c : 0u;
                    const uint2 q = *reinterpret_cast<const uint2 *>(lc + f_xo + cc * 64u);
                    const uint32_t sc = *reinterpret_cast<const uint32_t *>(ls + f_so + cc * 8u);
                    st.fx[u] = (kin & f_act) ? q : make_uint2(0, 0);
                    st.fxs[u] = (kin & f_sact) ? sc : 0u;
                }
                continue;
            }
            if (do_w) {
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    st.wq[u][j] = buf_load16(wcs, kin ? wco[j] + (uint32_t)c * cstep : kBufOOB);
                    st.wsc[u][j] = buf_load2(wss, kin ? wso[j] + (uint32_t)c * sstep : kBufOOB);
                }
            }
            if (!do_x) continue;
#pragma unroll
            for (int i = 0; i < MG; ++i) {
                if constexpr (kA == A_NVFP4) {
                    const uint32_t pc = xpo[i] + (uint32_t)c * (uint32_t)kPackBlock;
                    st.xq[u][i] = buf_load16(xcs, (kin & xv[i]) ? (apk ? pc : xco[i] + kc) : kBufOOB);
                    st.xsc[u][i] = buf_load2(xss, (kin & xv[i]) ? (apk ? pc + xps : xso[i] + ksc) : kBufOOB);
                } else {  // LDS: clamp the address, zero by select
                    const uint32_t kk = kin ? kc : 0u, kks = kin ? ksc : 0u;
                    const uint4 q = *reinterpret_cast<const uint4 *>(lc + xco[i] + kk);
                    const uint32_t sc = *reinterpret_cast<const uint16_t *>(ls + xso[i] + kks);
                    st.xq[u][i] = (kin & xv[i]) ? q : make_uint4(0, 0, 0, 0);
                    st.xsc[u][i] = (kin & xv[i]) ? sc : 0u;
                }
            }
        }
    };
    auto load = [&](int64_t c0, NStage &st) __attribute__((always_inline)) { load_part(c0, st, true, true); };
    auto compute = [&](const NStage &st) __attribute__((always_inline)) {
        if constexpr (kF4) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint2 xv = st.fx[u];
                const i32x8_t a8 = {f_hi ? 0 : (int)xv.x, f_hi ? 0 : (int)xv.y, f_hi ? (int)xv.x : 0,
                                    f_hi ? (int)xv.y : 0, 0, 0, 0, 0};
                float sa4[4];
                sa4[0] = __builtin_amdgcn_cvt_f32_fp8((int)st.fxs[u], 0);
                sa4[1] = __builtin_amdgcn_cvt_f32_fp8((int)st.fxs[u], 1);
                sa4[2] = __builtin_amdgcn_cvt_f32_fp8((int)st.fxs[u], 2);
                sa4[3] = __builtin_amdgcn_cvt_f32_fp8((int)st.fxs[u], 3);
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    const uint4 q = st.wq[u][j];
                    const i32x8_t b8 = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                    const f4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, f4_t{0.f, 0.f, 0.f, 0.f},
                                                                                   4, 4, 0, 127, 0, 127);
                    const float sw0 = __builtin_amdgcn_cvt_f32_fp8((int)st.fws[u][j], 0);
                    const float sw1 = __builtin_amdgcn_cvt_f32_fp8((int)st.fws[u][j], 1);
                    const float sw2 = __builtin_amdgcn_cvt_f32_fp8((int)st.fws[u][j], 2);
                    const float sw3 = __builtin_amdgcn_cvt_f32_fp8((int)st.fws[u][j], 3);
                    acc[0][j][0] = __builtin_fmaf(p[0], sa4[0] * sw0, acc[0][j][0]);
                    acc[0][j][1] = __builtin_fmaf(p[1], sa4[1] * sw1, acc[0][j][1]);
                    acc[0][j][2] = __builtin_fmaf(p[2], sa4[2] * sw2, acc[0][j][2]);
                    acc[0][j][3] = __builtin_fmaf(p[3], sa4[3] * sw3, acc[0][j][3]);
                }
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                half8_t b[NG];
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    const uint4 q = st.wq[u][j];
                    const uint32_t w = t == 0 ? q.x : t == 1 ? q.y : t == 2 ? q.z : q.w;
                    b[j] = expand8(w, e4m3_to_f16x2_over256(t < 2 ? (st.wsc[u][j] & 0xFFu) : (st.wsc[u][j] >> 8)));
                }
#pragma unroll
                for (int i = 0; i < MG; ++i) {
                    const uint4 q = st.xq[u][i];
                    const uint32_t xw = t == 0 ? q.x : t == 1 ? q.y : t == 2 ? q.z : q.w;
                    const half8_t a =
                        expand8(xw, e4m3_to_f16x2_over256(t < 2 ? (st.xsc[u][i] & 0xFFu) : (st.xsc[u][i] >> 8)));
#pragma unroll
                    for (int j = 0; j < NG; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[i][j], 0, 0, 0);
                }
            }
    };
    NStage s0, s1;
    if constexpr (kA != A_NVFP4) load_part(cs + wave, s0, true, false);
    if constexpr (kA != A_NVFP4) {
        // quantize the slice's part of the batch into LDS: codes [M][K/2],
        // then scales [M][K/16]
        extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
        uint8_t *lcw = xlds, *lsw = xlds + M * cb;
        // 32-bit indexing: M * K <= kFusedDecodeMaxElems
        const uint32_t octs = (uint32_t)(K >> 3), total = (uint32_t)M * octs;
        auto load_oct = [&](uint32_t r, uint32_t oc) __attribute__((always_inline)) {
            return *reinterpret_cast<const uint4 *>(x + (int64_t)r * ld_x + oc * 8);
        };
        auto oct_amax = [](const uint4 &v) __attribute__((always_inline)) {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            uint32_t am = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) am = max(am, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
            return am;
        };
        // alpha from this thread's partial amax (workgroup-wide reduction)
        auto set_alpha = [&](uint32_t am) __attribute__((always_inline)) {
            for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
            __shared__ uint32_t wmax[WAVES];
            if (lane == 0) wmax[wave] = am;
            __syncthreads();
            uint32_t t = wmax[0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v) t = max(t, wmax[v]);
            alpha_a = div_rn(bf16_bits_to_f32(t), kAlphaDen);
            if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a_alpha = alpha_a;
        };
        // Eq. 3 against t = alpha * 6 (one reciprocal per workgroup), Eq. 2 by
        // quant8_fast, or quant8 for a block outside its range, for octet oc
        // of row r held in v; thread pairs (t, t ^ 1) hold the two halves of
        // a 16-element block (every call site keeps octet parity = lane
        // parity), and `valid` is uniform across each pair.
        float at = 0.0f, art = 0.0f;
        auto quant_oct = [&](const uint4 &v, bool valid, uint32_t r, uint32_t oc) __attribute__((always_inline)) {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            const uint32_t am = oct_amax(v);
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false);
            const float amax_b = bf16_bits_to_f32(max(am, other));
            const uint32_t code = e4m3_encode(at > 0.0f ? div_rn_recip(amax_b, at, art) : 0.0f);
            const float d = alpha_a * e4m3_decode(code);
            const bool fast = d >= 0x1p-90f && d <= 0x1p100f && amax_b <= d * 0x1p120f;
            const uint32_t q = fast ? quant8_fast(w4, d, div_rn(1.0f, d)) : quant8(w4, d);
            if (valid) {
                *reinterpret_cast<uint32_t *>(lcw + r * cb + oc * 4) = q;
                if ((oc & 1) == 0) lsw[r * sb + (oc >> 1)] = (uint8_t)code;
            }
        };
        // batches of 3-8 rows (FP16 form) hold up to eight octets per thread;
        // the FP4 form (one or two rows) needs at most four
        constexpr uint32_t NT = WAVES * 64, kRegOcts = kF4 ? 4 : 8;
        const bool whole = cs == 0 && (uint32_t)ce * 16u >= octs;
        if (whole && total <= kRegOcts * NT) {
            // the batch fits in registers (kRegOcts octets per thread): one
            // load, the amax, then quantization from the same registers
            uint4 v[kRegOcts];
#pragma unroll
            for (uint32_t i = 0; i < kRegOcts; ++i) {
                const uint32_t o = threadIdx.x + i * NT, r = o < total ? o / octs : 0u;
                v[i] = o < total ? load_oct(r, o - r * octs) : make_uint4(0, 0, 0, 0);
            }
            if constexpr (kA == A_BF16_STATIC) {
                alpha_a = *a_alpha;
            } else {
                uint32_t am = 0;
#pragma unroll
                for (uint32_t i = 0; i < kRegOcts; ++i) am = max(am, oct_amax(v[i]));
                set_alpha(am);
            }
            at = alpha_a * kQmax;
            art = at > 0.0f ? div_rn(1.0f, at) : 0.0f;
#pragma unroll
            for (uint32_t i = 0; i < kRegOcts; ++i) {
                const uint32_t o = threadIdx.x + i * NT, r = o < total ? o / octs : 0u;
                if (i * NT < total) quant_oct(v[i], o < total, r, o - r * octs);  // wave-uniform condition
            }
        } else {
            if constexpr (kA == A_BF16_STATIC) {
                alpha_a = *a_alpha;
            } else {  // dynamic: the amax of the whole batch
                uint32_t am = 0;
                for (uint32_t o = threadIdx.x; o < total; o += NT) {
                    const uint32_t r = o / octs;
                    am = max(am, oct_amax(load_oct(r, o - r * octs)));
                }
                set_alpha(am);
            }
            at = alpha_a * kQmax;
            art = at > 0.0f ? div_rn(1.0f, at) : 0.0f;
            // the slice's octets of each row are [o0, o1); their count per row
            // is a multiple of 4 (K % 32 == 0), so pairs never straddle rows
            const uint32_t o0 = (uint32_t)cs * 16u, o1 = min((uint32_t)ce * 16u, octs), so = o1 - o0;
            const uint32_t stotal = (uint32_t)M * so;
            for (uint32_t base = 0; base < stotal; base += NT) {
                const uint32_t o = base + threadIdx.x;
                const uint32_t r = o < stotal ? o / so : 0u, oc = o < stotal ? o0 + (o - r * so) : 0u;
                quant_oct(o < stotal ? load_oct(r, oc) : make_uint4(0, 0, 0, 0), o < stotal, r, oc);
            }
        }
        __syncthreads();
        lc = lcw;
        ls = lsw;
    }

    const int64_t stride = (int64_t)WAVES * U;
    int64_t c0 = cs + wave;
    if constexpr (kA != A_NVFP4) load_part(c0, s0, false, true);  // the weights are in flight already
    else load(c0, s0);
    if constexpr (kPipe) {  // two chunk stages per trip, as in the BF16 decode kernel
        for (;;) {
            load(c0 + stride, s1);
            __builtin_amdgcn_sched_barrier(0);
            compute(s0);
            load(c0 + 2 * stride, s0);
            __builtin_amdgcn_sched_barrier(0);
            compute(s1);
            c0 += 2 * stride;
            if (c0 >= ce) break;
        }
    } else {  // the compiler's own schedule (faster for 4 x 4 tiles split over K)
        for (;;) {
            const int64_t c1 = c0 + stride;
            load(c1, s1);
            compute(s0);
            if (c1 >= ce) break;
            const int64_t c2 = c1 + stride;
            load(c2, s0);
            compute(s1);
            if (c2 >= ce) break;
            c0 = c2;
        }
    }

    if constexpr (kF4) {
        // a lane's four block sums, then the two lanes of its batch row
        // (blocks 0-3 and 4-7), into the 16x16 layout tile_reduce takes:
        // lanes 0-15 hold batch rows 0 and 1 of column n = lane
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float t = ((acc[0][j][0] + acc[0][j][1]) + acc[0][j][2]) + acc[0][j][3];
            t += __shfl_xor(t, 16);
            const float t1 = __shfl(t, (lane & 15) + 32);
            acc[0][j] = lane < 16 ? f4_t{t, t1, 0.f, 0.f} : f4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    float sa = 1.0f, sw = 1.0f;
    if constexpr (kOut != DOUT_PARTIAL) {
        sa = kA == A_NVFP4 ? *a_alpha : alpha_a;
        sw = *w_alpha;
    }
    tile_reduce<MG, NG, WAVES, kOut>(acc, sa, sw, M, N, n0, out, ld_out);
}

// Sum of the S partial tiles in slice order, then the epilogue
// y = (sum * alpha_A) * alpha_W (alphas absent: 1) into out [M, ld_out].
template <bool kOutBf16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int S, int64_t M,
                                                            int64_t N, const float *__restrict__ a_alpha,
                                                            const float *__restrict__ w_alpha, void *__restrict__ out,
                                                            int64_t ld_out) {
    const int64_t mn = M * N;
    const float sa = a_alpha ? *a_alpha : 1.0f, sw = w_alpha ? *w_alpha : 1.0f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += (int64_t)gridDim.x * 256) {
        float s = part[i];
        for (int j = 1; j < S; ++j) s += part[(int64_t)j * mn + i];
        const float y = (s * sa) * sw;
        const int64_t m = i / N, n = i - m * N;
        if (kOutBf16)
            reinterpret_cast<uint16_t *>(out)[m * ld_out + n] = (uint16_t)f32_to_bf16_bits(y);
        else
            reinterpret_cast<float *>(out)[m * ld_out + n] = y;
    }
}

hipError_t launch_reduce(const float *part, int S, int64_t M, int64_t N, const float *a_alpha, const float *w_alpha,
                         void *out, int out_type, int64_t ld_out, hipStream_t s) {
    const int64_t mn = M * N;
    int64_t g = (mn + 255) / 256;
    if (g > 4096) g = 4096;
    if (out_type == OUT_BF16)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, part, S, M, N, a_alpha,
                           w_alpha, out, ld_out);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, part, S, M, N, a_alpha,
                           w_alpha, out, ld_out);
    return hipGetLastError();
}

// Steps per slice for S slices of `steps` steps (S > 1 only while every
// slice keeps at least one step).
int64_t steps_per_slice(int64_t steps, int S) { return S <= 1 ? (steps > 0 ? steps : 1) : (steps + S - 1) / S; }

// BF16 decode kernel with NG column groups, WAVES waves, U steps per stage,
// S slices of K (S > 1: partials into `part`, then the reduction kernel);
// kPipe: the pinned two-stage loop, else the compiler's schedule.
template <int MG, int NG, int WAVES, int U, bool kPipe = true>
hipError_t launch_bf16_cfg(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                           int out_type, int64_t ld_out, int S, float *part, hipStream_t s, int packed) {
    const int64_t nb = (N + NG * 16 - 1) / (NG * 16);
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t sps = steps_per_slice((K + 31) >> 5, S);
    const int ns = S > 1 ? (int)((((K + 31) >> 5) + sps - 1) / sps) : 1;
    const dim3 grid((unsigned)nb, (unsigned)ns), block(WAVES * 64);
    if (ns > 1) {
        hipLaunchKernelGGL((skinny_kernel<MG, NG, WAVES, U, DOUT_PARTIAL, kPipe>), grid, block, 0, s, a, w, M, N, K,
                           (void *)part, N, sps, packed);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        return launch_reduce(part, ns, M, N, nullptr, nullptr, out, out_type, ld_out, s);
    }
    if (out_type == OUT_BF16)
        hipLaunchKernelGGL((skinny_kernel<MG, NG, WAVES, U, DOUT_BF16, kPipe>), grid, block, 0, s, a, w, M, N, K, out, ld_out,
                           sps, packed);
    else
        hipLaunchKernelGGL((skinny_kernel<MG, NG, WAVES, U, DOUT_F32, kPipe>), grid, block, 0, s, a, w, M, N, K, out, ld_out,
                           sps, packed);
    return hipGetLastError();
}

// NVFP4 decode kernel (kA: NVFP4 activations, or BF16 ones quantized inside;
// kF4: the FP4-MFMA form, for M <= 2 and K % 128 == 0; kPipe as above).
template <int MG, int NG, int WAVES, int U, int kA = A_NVFP4, bool kF4 = false, bool kPipe = true>
hipError_t launch_nvfp4_cfg(const uint8_t *ac, const uint8_t *as, float *aa, const uint8_t *wc, const uint8_t *ws,
                            const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                            int S, float *part, hipStream_t s, const uint16_t *x = nullptr, int64_t ld_x = 0,
                            int packed = 0) {
    const int64_t nb = (N + NG * 16 - 1) / (NG * 16);
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t chunks = (K + 127) >> 7, sps = steps_per_slice(chunks, S);
    const int ns = S > 1 ? (int)((chunks + sps - 1) / sps) : 1;
    const size_t lds = kA == A_NVFP4 ? 0 : (size_t)(M * K / 2 + M * K / 16);
    const int kind = ns > 1 ? DOUT_PARTIAL : out_type == OUT_BF16 ? DOUT_BF16 : DOUT_F32;
    const void *f = kind == DOUT_PARTIAL ? (const void *)skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_PARTIAL, kA, kF4, kPipe>
                    : kind == DOUT_BF16  ? (const void *)skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_BF16, kA, kF4, kPipe>
                                         : (const void *)skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_F32, kA, kF4, kPipe>;
    if (kA != A_NVFP4) {
        static std::atomic<uint32_t> attr_done[3];
        if (hipError_t e = set_dyn_lds_once(attr_done[kind], f, (int)(kFusedDecodeMaxElems * 9 / 16)); e != hipSuccess)
            return e;
    }
    const dim3 grid((unsigned)nb, (unsigned)ns), block(WAVES * 64);
    void *dst = ns > 1 ? (void *)part : out;
    const int64_t ld = ns > 1 ? N : ld_out;
    if (kind == DOUT_PARTIAL)
        hipLaunchKernelGGL((skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_PARTIAL, kA, kF4, kPipe>), grid, block, lds, s, ac, as, aa,
                           wc, ws, wa, M, N, K, dst, ld, x, ld_x, sps, packed);
    else if (kind == DOUT_BF16)
        hipLaunchKernelGGL((skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_BF16, kA, kF4, kPipe>), grid, block, lds, s, ac, as, aa, wc,
                           ws, wa, M, N, K, dst, ld, x, ld_x, sps, packed);
    else
        hipLaunchKernelGGL((skinny_nvfp4_kernel<MG, NG, WAVES, U, DOUT_F32, kA, kF4, kPipe>), grid, block, lds, s, ac, as, aa, wc,
                           ws, wa, M, N, K, dst, ld, x, ld_x, sps, packed);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (ns > 1) return launch_reduce(part, ns, M, N, aa, wa, out, out_type, ld_out, s);
    return hipSuccess;
}

// Decode-packed weights: one wave per (16-row group, 128-wide chunk) block;
// lane l copies the 16 code bytes lane l of a decode wave loads, lanes 0-15
// the 8 scale bytes of row 16 g + l; rows past N are written as zeros.
__global__ __launch_bounds__(256) void decode_pack_kernel(const uint8_t *__restrict__ wc,
                                                          const uint8_t *__restrict__ ws, int64_t N, int64_t K,
                                                          uint8_t *__restrict__ wp, int64_t blocks) {
    const int lane = threadIdx.x & 63;
    const int64_t chunks = K >> 7;
    for (int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < blocks; b += (int64_t)gridDim.x * 4) {
        const int64_t g = b / chunks, c = b - g * chunks;
        const int64_t row = g * 16 + (lane & 15);
        uint4 q = make_uint4(0, 0, 0, 0);
        if (row < N) q = *reinterpret_cast<const uint4 *>(wc + row * (K >> 1) + c * 64 + (lane >> 4) * 16);
        uint8_t *blk = wp + b * kPackBlock;
        *reinterpret_cast<uint4 *>(blk + lane * 16) = q;
        if (lane < 16) {
            uint2 sc = make_uint2(0, 0);
            if (row < N) {
                const uint32_t *sp = reinterpret_cast<const uint32_t *>(ws + row * (K >> 4) + c * 8);
                sc = make_uint2(sp[0], sp[1]);
            }
            *reinterpret_cast<uint2 *>(blk + 1024 + lane * 8) = sc;
        }
    }
}

// BF16 decode-packed weights: one wave per (16-row group, 32-wide K step)
// block of 1 KB; lane l copies the 16 bytes lane l of a decode wave loads
// (row 16 g + l % 16, elements 32 t + 8 (l / 16) .. + 7); rows past N are zeros.
__global__ __launch_bounds__(256) void bf16_pack_kernel(const uint16_t *__restrict__ w, int64_t N, int64_t K,
                                                        uint8_t *__restrict__ wp, int64_t blocks) {
    const int lane = threadIdx.x & 63;
    const int64_t steps = K >> 5;
    for (int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < blocks; b += (int64_t)gridDim.x * 4) {
        const int64_t g = b / steps, t = b - g * steps;
        const int64_t row = g * 16 + (lane & 15);
        uint4 q = make_uint4(0, 0, 0, 0);
        if (row < N) q = *reinterpret_cast<const uint4 *>(w + row * K + t * 32 + (lane >> 4) * 8);
        *reinterpret_cast<uint4 *>(wp + b * 1024 + lane * 16) = q;
    }
}

__global__ void fill_zero_kernel(uint8_t *out, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
        for (int64_t c = threadIdx.x; c < row_bytes; c += blockDim.x) out[r * ld_bytes + c] = 0;
}

}  // namespace

// Decode plan: column groups per workgroup (ng), waves per workgroup, K steps
// per register stage (u) and K slices (s), from a sweep of every
// configuration over the Qwen3-8B projections at batch 1-64 (graph replay,
// rotated weights).  Batches up to 16 are fastest unsplit; larger ones split
// K so that narrow layers still give about 256 workgroups of wide strips
// (BF16), or, for NVFP4 whose weights are 3.6x smaller, only on long K.
// Strip width (16-column groups) among `cands` whose s * ceil(N / (16 ng))
// workgroups best fill whole rounds of one workgroup per CU on the 256 CUs of
// an MI355X (ties: the wider strip, which re-reads the batch less often).
static int fill_ng(int64_t N, int s, std::initializer_list<int> cands) {
    int best = 0;
    double best_fill = -1.0;
    for (int ng : cands) {
        const int64_t wgs = s * ((N + 16 * ng - 1) / (16 * ng)), rounds = (wgs + 255) / 256;
        const double fill = (double)wgs / (double)(rounds * 256);
        if (fill > best_fill + 1e-9 || (fill > best_fill - 1e-9 && ng > best)) {
            best = ng;
            best_fill = fill;
        }
    }
    return best;
}

DecodePlan decode_plan(int kind, int64_t M, int64_t N, int64_t K) {
    // the FP4-MFMA form of the NVFP4 kernel (M <= 2, K % 128 == 0), from its
    // own sweep (fused and unfused, batch 1 and 2): narrower strips and fewer
    // waves than the FP16-expansion form, two chunks per register stage
    if (kind != DECODE_BF16 && decode_fp4_form(M, K)) {
        // wide layers: two 16-row groups per workgroup (gate_up on
        // decode-packed weights, fused batch 1: 15.5 -> 14.0 us; the K
        // order, set by waves and chunks per stage, is unchanged)
        if (N >= 16384) return {2, 4, 2, 1};
        if (K >= 8192) return {1, 16, 1, 1};
        return {1, 8, 2, 1};
    }
    // pipe = false (the compiler's schedule of the K loop) where it measured
    // faster: one column group of 16 waves (BF16: batch 1 qkv / o / down
    // 13.6 / 8.2 / 21.4 us against 13.9 / 8.9 / 23.8 with the pinned loop)
    // and 4 x 4 NVFP4 tiles split over K (down at batch 64: 24.8 against 26.9)
    if (kind == DECODE_BF16) {
        // 6144-16383 columns at batch <= 16: 32-column strips of 4 waves, four
        // steps per stage (qkv on decode-packed weights, batch 1: 12.6 -> 11.1 us)
        if (M <= 16 && N >= 6144 && N < 16384) return {2, 4, 4, 1};
        if (M <= 4) return {1, 16, 1, 1, false};
        // wide layers at batch 5-16: the same 32-column strips of 4 waves
        // (gate_up at batch 8 on decode-packed weights, four-layer step
        // 80.4 -> 78.8 us against 16 waves)
        if (M <= 16) return N >= 6144 ? DecodePlan{2, 4, 4, 1} : DecodePlan{1, 16, 1, 1, false};
        // wide layers at batch 33-64: wide strips read the batch once per 64-128
        // columns (gate_up at batch 64: 77.9 -> 69.8 us with 128-column strips
        // instead of 64), and a width that fills whole rounds of the CUs
        // (96 columns, 256 workgroups for gate_up on decode-packed weights:
        // 52.0 -> 46.8 us)
        if (M > 32 && N >= 16384) return {fill_ng(N, 1, {4, 6, 8}), 4, 1, 1};
        const int ng = N >= 6144 || M > 32 ? 4 : 2;
        const int64_t nb = (N + 16 * ng - 1) / (16 * ng);
        const int s = nb <= 64 ? 4 : 2;
        if (ng == 2) return DecodePlan{2, 8, 1, s};
        // 48-column strips where they fill the CUs better (qkv at batch 64,
        // two K slices: 256 workgroups instead of 192, 23.0 -> 20.6 us)
        return DecodePlan{M > 32 && s == 2 ? fill_ng(N, 2, {3, 4}) : 4, 4, 2, s};
    }
    // NVFP4 and fused: the same plan, so both sum in the same order
    if (M <= 16) return N >= 6144 ? DecodePlan{2, 8, 1, 1} : DecodePlan{1, 16, 1, 1};
    // batch 33-64 with the activation in the packed block layout (the
    // quantize-first route of nvfp4_quant_gemm): narrow and long-K layers
    // take one 16-column group of 16 waves, unsplit (down at batch 64 on
    // decode-packed weights 26.4 -> 23.8 us against 4 groups over 4 K
    // slices, o 15.4 -> 14.9 us against 8 waves of two chunks per stage)
    if (K >= 8192) return M > 32 ? DecodePlan{1, 16, 1, 1} : DecodePlan{4, 8, 1, 4, false};
    // wide layers at batch 33-64: 4 waves, strips that fill whole rounds of
    // the CUs (gate_up at batch 64 on decode-packed weights: 96-column strips,
    // 256 workgroups, 25.7 us against 36.0 with 32-column strips of 768)
    if (N >= 16384 && M > 32) return {fill_ng(N, 1, {4, 6, 8}), 4, 1, 1};
    if (N >= 6144) return {2, 8, 1, 1};
    return M > 32 ? DecodePlan{1, 16, 1, 1} : DecodePlan{1, 8, 2, 1};
}

size_t decode_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K) {
    const DecodePlan p = decode_plan(kind, M, N, K);
    return p.s > 1 ? (size_t)p.s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

namespace {

// the plan's slice count when the workspace holds its partials, else 1
int plan_slices(const DecodePlan &p, int64_t M, int64_t N, void *ws, size_t ws_bytes) {
    const size_t need = (size_t)p.s * (size_t)M * (size_t)N * sizeof(float);
    return p.s > 1 && ws && ws_bytes >= need ? p.s : 1;
}

template <int MG>
hipError_t launch_bf16_mg(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                          int out_type, int64_t ld_out, const DecodePlan &p, int S, float *part, hipStream_t s,
                          int pk) {
    if (p.ng == 8) return launch_bf16_cfg<MG, 8, 4, 1>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    if constexpr (MG == 4) {
        if (p.ng == 6) return launch_bf16_cfg<4, 6, 4, 1>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
        if (p.ng == 3) return launch_bf16_cfg<4, 3, 4, 2>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    }
    if (p.ng == 4) return launch_bf16_cfg<MG, 4, 4, 2>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    if (p.ng == 2 && p.waves == 8) return launch_bf16_cfg<MG, 2, 8, 1>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    if constexpr (MG == 1)
        if (p.ng == 2 && p.waves == 4) return launch_bf16_cfg<1, 2, 4, 4>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    if (p.ng == 2) return launch_bf16_cfg<MG, 2, 16, 1>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    if constexpr (MG == 1)
        if (!p.pipe) return launch_bf16_cfg<1, 1, 16, 1, false>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
    return launch_bf16_cfg<MG, 1, 16, 1>(a, w, M, N, K, out, out_type, ld_out, S, part, s, pk);
}

// The FP4-MFMA form (M <= 2, K % 128 == 0) of the plans decode_plan gives it.
template <int kA>
hipError_t launch_f4(const uint8_t *ac, const uint8_t *as, float *aa, const uint8_t *wc, const uint8_t *ws,
                     const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                     const DecodePlan &p, int S, float *part, hipStream_t s, const uint16_t *x, int64_t ld_x, int pk) {
    if (p.waves == 4 && p.ng == 2)
        return launch_nvfp4_cfg<1, 2, 4, 2, kA, true>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                      x, ld_x, pk);
    if (p.waves == 4)
        return launch_nvfp4_cfg<1, 1, 4, 2, kA, true>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                      x, ld_x, pk);
    if (p.waves == 8)
        return launch_nvfp4_cfg<1, 1, 8, 2, kA, true>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                      x, ld_x, pk);
    return launch_nvfp4_cfg<1, 1, 16, 1, kA, true>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                   x, ld_x, pk);
}

template <int MG>
hipError_t launch_nv_mg(const uint8_t *ac, const uint8_t *as, const float *aa_in, const uint8_t *wc,
                        const uint8_t *ws, const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                        int64_t ld_out, const DecodePlan &p, int S, float *part, hipStream_t s, int pk) {
    float *aa = const_cast<float *>(aa_in);  // only read when A is NVFP4
    if constexpr (MG == 1)
        if (decode_fp4_form(M, K))
            return launch_f4<A_NVFP4>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, p, S, part, s, nullptr, 0,
                                      pk);
    if constexpr (MG == 4)
        if (p.waves == 4) {  // wide layers at batch 33-64
            if (p.ng == 4)
                return launch_nvfp4_cfg<4, 4, 4, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                    nullptr, 0, pk);
            if (p.ng == 6)
                return launch_nvfp4_cfg<4, 6, 4, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                    nullptr, 0, pk);
            return launch_nvfp4_cfg<4, 8, 4, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                nullptr, 0, pk);
        }
    if (p.ng == 4 && !p.pipe)
        return launch_nvfp4_cfg<MG, 4, 8, 1, A_NVFP4, false, false>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type,
                                                                    ld_out, S, part, s, nullptr, 0, pk);
    if (p.ng == 4) return launch_nvfp4_cfg<MG, 4, 8, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                       nullptr, 0, pk);
    if (p.ng == 2) return launch_nvfp4_cfg<MG, 2, 8, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                       nullptr, 0, pk);
    if (p.waves == 8)
        return launch_nvfp4_cfg<MG, 1, 8, 2>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                       nullptr, 0, pk);
    return launch_nvfp4_cfg<MG, 1, 16, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, S, part, s,
                                                       nullptr, 0, pk);
}

template <int kA>
hipError_t launch_fused_a(const uint16_t *x, int64_t ld_x, float *a_alpha, const uint8_t *wc, const uint8_t *ws,
                          const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                          const DecodePlan &p, int S, float *part, hipStream_t s, int pk) {
    if (decode_fp4_form(M, K))
        return launch_f4<kA>(nullptr, nullptr, a_alpha, wc, ws, wa, M, N, K, out, out_type, ld_out, p, S, part, s, x,
                             ld_x, pk);
    if (p.ng == 2)
        return launch_nvfp4_cfg<1, 2, 8, 1, kA>(nullptr, nullptr, a_alpha, wc, ws, wa, M, N, K, out, out_type, ld_out, S,
                                                part, s, x, ld_x, pk);
    return launch_nvfp4_cfg<1, 1, 16, 1, kA>(nullptr, nullptr, a_alpha, wc, ws, wa, M, N, K, out, out_type, ld_out, S,
                                             part, s, x, ld_x, pk);
}

}  // namespace

hipError_t launch_skinny_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                              int out_type, int64_t ld_out, void *ws, size_t ws_bytes, hipStream_t s, bool packed) {
    const DecodePlan p = decode_plan(DECODE_BF16, M, N, K);
    const int S = plan_slices(p, M, N, ws, ws_bytes);
    float *part = (float *)ws;
    if (M <= 16) return launch_bf16_mg<1>(a, w, M, N, K, out, out_type, ld_out, p, S, part, s, packed);
    if (M <= 32) return launch_bf16_mg<2>(a, w, M, N, K, out, out_type, ld_out, p, S, part, s, packed);
    if (M <= 64) return launch_bf16_mg<4>(a, w, M, N, K, out, out_type, ld_out, p, S, part, s, packed);
    return hipErrorInvalidValue;
}

hipError_t launch_skinny_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                               int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, void *ws,
                               size_t ws_bytes, hipStream_t s, int packed) {
    if ((packed & kPackA) && (decode_fp4_form(M, K) || K % 128 != 0)) return hipErrorInvalidValue;
    const DecodePlan p = decode_plan(DECODE_NVFP4, M, N, K);
    const int S = plan_slices(p, M, N, ws, ws_bytes);
    float *part = (float *)ws;
    if (M <= 16)
        return launch_nv_mg<1>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out,
                               p, S, part, s, packed);
    if (M <= 32)
        return launch_nv_mg<2>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out,
                               p, S, part, s, packed);
    if (M <= 64)
        return launch_nv_mg<4>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out,
                               p, S, part, s, packed);
    return hipErrorInvalidValue;
}

hipError_t launch_skinny_fused(const uint16_t *x, int64_t ld_x, float *a_alpha, int dynamic, const uint8_t *w_codes,
                               const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                               void *out, int out_type, int64_t ld_out, void *ws, size_t ws_bytes, hipStream_t s,
                               bool packed) {
    if (M > 16 || M * K > kFusedDecodeMaxElems) return hipErrorInvalidValue;
    const DecodePlan p = decode_plan(DECODE_FUSED, M, N, K);
    const int S = plan_slices(p, M, N, ws, ws_bytes);
    float *part = (float *)ws;
    if (dynamic)
        return launch_fused_a<A_BF16_DYNAMIC>(x, ld_x, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type,
                                              ld_out, p, S, part, s, packed);
    return launch_fused_a<A_BF16_STATIC>(x, ld_x, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out,
                                         p, S, part, s, packed);
}

hipError_t launch_decode_pack(const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, int64_t K,
                              uint8_t *w_packed, hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    if (K % 128 != 0) return hipErrorInvalidValue;
    const int64_t blocks = ((N + 15) / 16) * (K / 128);
    int64_t g = (blocks + 3) / 4;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(decode_pack_kernel, dim3((unsigned)g), dim3(256), 0, s, w_codes, w_scales, N, K, w_packed,
                       blocks);
    return hipGetLastError();
}

hipError_t launch_bf16_pack(const uint16_t *w, int64_t N, int64_t K, uint8_t *w_packed, hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    if (K % 32 != 0) return hipErrorInvalidValue;
    const int64_t blocks = ((N + 15) / 16) * (K / 32);
    int64_t g = (blocks + 3) / 4;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(bf16_pack_kernel, dim3((unsigned)g), dim3(256), 0, s, w, N, K, w_packed, blocks);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *out, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t g = rows < 4096 ? rows : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s, (uint8_t *)out, rows, cols * elem_bytes,
                       ld * elem_bytes);
    return hipGetLastError();
}

}  // namespace nvfp4
