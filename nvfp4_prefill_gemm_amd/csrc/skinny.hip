// Decode-shape GEMMs for small batches (M <= 64): Y[M, N] = X[M, K] * W[N, K]^T.
//
// BF16: decode keeps the original BF16 weights (Mix-Quant Section 3.3,
// "Prefill-Decode Disaggregation Deployment") and is bound by streaming W
// from HBM: 2*N*K bytes against 2*M*N*K flops.  Each workgroup owns a strip
// of NG*16 weight rows; its waves split K in 32-wide steps (interleaved, so
// the waves of a workgroup read neighbouring 64-byte pieces of the same
// rows), load through buffer resources over the valid rows (steps past K and
// rows past N or M read zeros, so the loop has no branches), keep two
// register stages of U steps in flight, and run 16x16x32 BF16 MFMAs with X
// zero-padded to MG*16 rows.  The per-wave partial tiles are summed through
// LDS at the end.
//
// NVFP4 (both operands E2M1 + E4M3 per 16, the uniform-NVFP4 and
// FP4-decode variants of Mix-Quant's ablations, Section 4): the same split-K
// layout streams 0.5625 bytes per weight instead of 2.  A lane's 16-byte code
// load covers 32 consecutive K; the four 16x16x32 MFMA sub-steps of a
// 128-wide K chunk take its four 8-code words, so sub-step t of lane group g
// holds K = 128c + 32g + 8t + i on both operands (the same permutation of K
// for A and W, which leaves the dot product unchanged).  Codes are expanded
// exactly to q * sigma in FP16 in registers; alpha_A * alpha_W is applied in
// the epilogue as in the prefill GEMM.
//
// Fused decode (nvfp4_quant_gemm with M * K <= 196608): the workgroup first
// quantizes the BF16 batch itself, one 8-element group per thread with the
// quantizer's own Eq. 3 / Eq. 2 functions, into LDS (a dynamic tensor scale
// is formed from a first pass over the batch; every workgroup derives the
// same alpha_A and workgroup 0 stores it), then runs the loop above with the
// activation codes read from LDS.  Codes, scales and the summation order
// equal those of quantize followed by the decode GEMM, so the two paths agree
// bit for bit.
#include <stdlib.h>
#include <string.h>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(4))) float f4_t;

// Sum the per-wave 16x16 partial tiles of a workgroup through LDS, one
// (row group, column group) tile at a time, and store y = (sum * sa) * sw:
// out[m = i*16 + (l>>4)*4 + r][n = n0 + j*16 + (l & 15)].
template <int MG, int NG, int WAVES, bool kOutBf16>
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
                const float y = (s * sa) * sw;
                const int64_t m = i * 16 + (l >> 4) * 4 + r, n = n0 + j * 16 + (l & 15);
                if (m < M && n < N) {
                    if (kOutBf16)
                        reinterpret_cast<uint16_t *>(out)[m * ld_out + n] = (uint16_t)f32_to_bf16_bits(y);
                    else
                        reinterpret_cast<float *>(out)[m * ld_out + n] = y;
                }
            }
        }
}

template <int MG, int NG, int WAVES, int U, bool kOutBf16>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                            int64_t M, int64_t N, int64_t K, void *__restrict__ out,
                                                            int64_t ld_out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * (NG * 16);
    const int kq = (lane >> 4) * 8;
    const int64_t KS = (K + 31) >> 5;

    f4_t acc[MG][NG];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    // buffer resources over this workgroup's weight rows and over X: rows past
    // N or M and steps past K read zeros (offset beyond the resource)
    const int64_t nrows = N - n0 < NG * 16 ? N - n0 : NG * 16;
    const rsrc_t wrs = make_rsrc(w + n0 * K, (uint32_t)(nrows * K * 2));
    const rsrc_t xrs = make_rsrc(x, (uint32_t)(M * K * 2));
    uint32_t wro[NG], xro[MG];  // byte offsets of this lane's rows
#pragma unroll
    for (int j = 0; j < NG; ++j) wro[j] = (uint32_t)((j * 16 + (lane & 15)) * K * 2);
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
            const int64_t k = (ks0 + (int64_t)u * WAVES) * 32 + kq;
            const bool kin = k + 8 <= K;  // also false past the last step
#pragma unroll
            for (int j = 0; j < NG; ++j) bw[u][j] = buf_load16(wrs, kin ? wro[j] + (uint32_t)(k * 2) : kBufOOB);
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
    int64_t ks0 = wave;
    load(ks0, bw0, ax0);
    for (;;) {
        const int64_t k1 = ks0 + stride;
        load(k1, bw1, ax1);
        compute(bw0, ax0);
        if (k1 >= KS) break;
        const int64_t k2 = k1 + stride;
        load(k2, bw0, ax0);
        compute(bw1, ax1);
        if (k2 >= KS) break;
        ks0 = k2;
    }

    tile_reduce<MG, NG, WAVES, kOutBf16>(acc, 1.0f, 1.0f, M, N, n0, out, ld_out);
}

template <int MG, int NG, int WAVES, int U>
hipError_t launch_cfg(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                      int64_t ld_out, hipStream_t s) {
    const int64_t nb = (N + NG * 16 - 1) / (NG * 16);
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (out_type == OUT_BF16)
        hipLaunchKernelGGL((skinny_kernel<MG, NG, WAVES, U, true>), dim3((unsigned)nb), dim3(WAVES * 64), 0, s, a, w,
                           M, N, K, out, ld_out);
    else
        hipLaunchKernelGGL((skinny_kernel<MG, NG, WAVES, U, false>), dim3((unsigned)nb), dim3(WAVES * 64), 0, s, a, w,
                           M, N, K, out, ld_out);
    return hipGetLastError();
}

// Source of the A operand of the decode kernel.
enum ASrc { A_NVFP4 = 0, A_BF16_DYNAMIC = 1, A_BF16_STATIC = 2 };

// NVFP4 x NVFP4, M <= MG*16, NG*16 weight rows per workgroup, K % 32 == 0,
// 16-byte aligned codes and 4-byte aligned scales.  kA != A_NVFP4: A is
// BF16 [M, ld_x] (16-byte aligned rows, MG == 1), quantized into LDS
// (M * K * 9 / 16 bytes of dynamic shared memory).
template <int MG, int NG, int WAVES, int U, bool kOutBf16, int kA = A_NVFP4>
__global__ __launch_bounds__(WAVES * 64) void skinny_nvfp4_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, float *__restrict__ a_alpha,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, const float *__restrict__ w_alpha, int64_t M,
    int64_t N, int64_t K, void *__restrict__ out, int64_t ld_out, const uint16_t *__restrict__ x, int64_t ld_x) {
    static_assert(kA == A_NVFP4 || MG == 1, "BF16 activations: one 16-row group");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * (NG * 16);
    const int64_t cb = K >> 1, sb = K >> 4;  // code and scale bytes per row
    const int64_t KC = (K + 127) >> 7;       // 128-wide K chunks
    const int kg = (lane >> 4) * 32;         // this lane group's K offset in a chunk

    f4_t acc[MG][NG];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    // buffer resources over this workgroup's weight rows (and over A in global
    // memory): rows past N or M and chunks past K read zeros
    const int64_t nrows = N - n0 < NG * 16 ? N - n0 : NG * 16;
    const rsrc_t wcs = make_rsrc(wc + n0 * cb, (uint32_t)(nrows * cb));
    const rsrc_t wss = make_rsrc(ws + n0 * sb, (uint32_t)(nrows * sb));
    const rsrc_t xcs = make_rsrc(ac, (uint32_t)(M * cb));
    const rsrc_t xss = make_rsrc(as, (uint32_t)(M * sb));
    uint32_t wco[NG], wso[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        wco[j] = (uint32_t)((j * 16 + (lane & 15)) * cb);
        wso[j] = (uint32_t)((j * 16 + (lane & 15)) * sb);
    }
    uint32_t xco[MG], xso[MG];
    bool xv[MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) {
        const int64_t m = i * 16 + (lane & 15);
        xv[i] = m < M;
        xco[i] = (uint32_t)((xv[i] ? m : 0) * cb);
        xso[i] = (uint32_t)((xv[i] ? m : 0) * sb);
    }
    const uint8_t *lc = nullptr, *ls = nullptr;  // LDS copy of A (fused path)
    float alpha_a = 0.0f;
    // Two register stages of U chunks each, as in the BF16 decode kernel.
    struct NStage {
        uint4 wq[U][NG], xq[U][MG];
        uint32_t wsc[U][NG], xsc[U][MG];
    };
    // weights (w) and the batch (x) of a stage; the fused path issues the
    // first stage's weight loads before it quantizes the batch
    auto load_part = [&](int64_t c0, NStage &st, bool do_w, bool do_x) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = (c0 + (int64_t)u * WAVES) * 128 + kg;
            const bool kin = k < K;  // K % 32 == 0: the lane's 32 codes are all in or all out
            const uint32_t kc = (uint32_t)(k >> 1), ksc = (uint32_t)(k >> 4);
            if (do_w) {
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    st.wq[u][j] = buf_load16(wcs, kin ? wco[j] + kc : kBufOOB);
                    st.wsc[u][j] = buf_load2(wss, kin ? wso[j] + ksc : kBufOOB);
                }
            }
            if (!do_x) continue;
#pragma unroll
            for (int i = 0; i < MG; ++i) {
                if constexpr (kA == A_NVFP4) {
                    st.xq[u][i] = buf_load16(xcs, (kin & xv[i]) ? xco[i] + kc : kBufOOB);
                    st.xsc[u][i] = buf_load2(xss, (kin & xv[i]) ? xso[i] + ksc : kBufOOB);
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
    if constexpr (kA != A_NVFP4) load_part(wave, s0, true, false);
    if constexpr (kA != A_NVFP4) {
        // quantize the whole batch into LDS: codes [M][K/2], then scales [M][K/16]
        extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];
        uint8_t *lcw = xlds, *lsw = xlds + M * cb;
        // 32-bit indexing: M * K <= kFusedDecodeMaxElems
        const uint32_t octs = (uint32_t)(K >> 3), total = (uint32_t)M * octs;  // total is even (K % 32 == 0)
        auto load_oct = [&](uint32_t o) __attribute__((always_inline)) {
            if (o >= total) return make_uint4(0, 0, 0, 0);
            const uint32_t r = o / octs;
            return *reinterpret_cast<const uint4 *>(x + (int64_t)r * ld_x + (o - r * octs) * 8);
        };
        if constexpr (kA == A_BF16_STATIC) {
            alpha_a = *a_alpha;
        } else {
            uint32_t am = 0;
            for (uint32_t o = threadIdx.x; o < total; o += WAVES * 64) {
                const uint4 v = load_oct(o);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) am = max(am, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
            }
            for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
            __shared__ uint32_t wmax[WAVES];
            if (lane == 0) wmax[wave] = am;
            __syncthreads();
            uint32_t t = wmax[0];
#pragma unroll
            for (int v = 1; v < WAVES; ++v) t = max(t, wmax[v]);
            alpha_a = div_rn(bf16_bits_to_f32(t), kAlphaDen);
            if (blockIdx.x == 0 && threadIdx.x == 0) *a_alpha = alpha_a;
        }
        // Eq. 3 against t = alpha * 6 (one reciprocal per workgroup), Eq. 2 by
        // quant8_fast, or quant8 for a block outside its range
        const float at = alpha_a * kQmax, art = at > 0.0f ? div_rn(1.0f, at) : 0.0f;
        // thread pairs (t, t ^ 1) hold the two halves of a 16-element block
        for (uint32_t base = 0; base < total; base += WAVES * 64) {
            const uint32_t o = base + threadIdx.x;
            const uint4 v = load_oct(o);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            uint32_t am = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) am = max(am, max(w4[e] & 0x7FFFu, (w4[e] >> 16) & 0x7FFFu));
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false);
            const float amax_b = bf16_bits_to_f32(max(am, other));
            const uint32_t code = e4m3_encode(at > 0.0f ? div_rn_recip(amax_b, at, art) : 0.0f);
            const float d = alpha_a * e4m3_decode(code);
            const bool fast = d >= 0x1p-90f && d <= 0x1p100f && amax_b <= d * 0x1p120f;
            const uint32_t q = fast ? quant8_fast(w4, d, div_rn(1.0f, d)) : quant8(w4, d);
            if (o < total) {
                const uint32_t r = o / octs, oc = o - r * octs;
                *reinterpret_cast<uint32_t *>(lcw + r * cb + oc * 4) = q;
                if ((oc & 1) == 0) lsw[r * sb + (oc >> 1)] = (uint8_t)code;
            }
        }
        __syncthreads();
        lc = lcw;
        ls = lsw;
    }

    const int64_t stride = (int64_t)WAVES * U;
    int64_t c0 = wave;
    if constexpr (kA != A_NVFP4) load_part(c0, s0, false, true);  // the weights are in flight already
    else load(c0, s0);
    for (;;) {
        const int64_t c1 = c0 + stride;
        load(c1, s1);
        compute(s0);
        if (c1 >= KC) break;
        const int64_t c2 = c1 + stride;
        load(c2, s0);
        compute(s1);
        if (c2 >= KC) break;
        c0 = c2;
    }

    tile_reduce<MG, NG, WAVES, kOutBf16>(acc, kA == A_NVFP4 ? *a_alpha : alpha_a, *w_alpha, M, N, n0, out, ld_out);
}

template <int MG, int NG, int WAVES, int U, int kA = A_NVFP4>
hipError_t launch_nvfp4_cfg(const uint8_t *ac, const uint8_t *as, float *aa, const uint8_t *wc, const uint8_t *ws,
                            const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type, int64_t ld_out,
                            hipStream_t s, const uint16_t *x = nullptr, int64_t ld_x = 0) {
    const int64_t nb = (N + NG * 16 - 1) / (NG * 16);
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = kA == A_NVFP4 ? 0 : (size_t)(M * K / 2 + M * K / 16);
    if (kA != A_NVFP4) {
        static std::atomic<uint32_t> attr_done[2];
        const int o = out_type == OUT_BF16;
        const void *f = o ? (const void *)skinny_nvfp4_kernel<MG, NG, WAVES, U, true, kA>
                          : (const void *)skinny_nvfp4_kernel<MG, NG, WAVES, U, false, kA>;
        if (hipError_t e = set_dyn_lds_once(attr_done[o], f, (int)(kFusedDecodeMaxElems * 9 / 16)); e != hipSuccess)
            return e;
    }
    if (out_type == OUT_BF16)
        hipLaunchKernelGGL((skinny_nvfp4_kernel<MG, NG, WAVES, U, true, kA>), dim3((unsigned)nb), dim3(WAVES * 64),
                           lds, s, ac, as, aa, wc, ws, wa, M, N, K, out, ld_out, x, ld_x);
    else
        hipLaunchKernelGGL((skinny_nvfp4_kernel<MG, NG, WAVES, U, false, kA>), dim3((unsigned)nb), dim3(WAVES * 64),
                           lds, s, ac, as, aa, wc, ws, wa, M, N, K, out, ld_out, x, ld_x);
    return hipGetLastError();
}

__global__ void fill_zero_kernel(uint8_t *out, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
        for (int64_t c = threadIdx.x; c < row_bytes; c += blockDim.x) out[r * ld_bytes + c] = 0;
}

}  // namespace

// NVFP4_SKINNY_CFG=8|16 overrides the waves per workgroup of the BF16 decode
// kernel with one column group (tuning knob; default 16).
int skinny_cfg() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("NVFP4_SKINNY_CFG");
        v = (e && !strcmp(e, "8")) ? 1 : 0;
    }
    return v;
}

// K-steps per register stage.  With one row group a single step per stage
// (two steps in flight per wave) measured fastest on the Qwen3-8B decode
// layers; more row groups take two.
template <int MG>
constexpr int skinny_u() { return MG == 1 ? 1 : 2; }

template <int MG, int NG>
hipError_t launch_mg(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                     int64_t ld_out, hipStream_t s) {
    if (skinny_cfg() == 1) return launch_cfg<MG, NG, 8, skinny_u<MG>()>(a, w, M, N, K, out, out_type, ld_out, s);
    return launch_cfg<MG, NG, 16, skinny_u<MG>()>(a, w, M, N, K, out, out_type, ld_out, s);
}

// NVFP4_DECODE_NG=1|2|4 forces the number of 16-column groups per
// workgroup (tuning knob); by default it follows the layer width below.
int decode_ng_knob() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("NVFP4_DECODE_NG");
        v = e ? atoi(e) : 0;
        if (v != 1 && v != 2 && v != 4) v = 0;
    }
    return v;
}

// With several 16-row groups of X, each X fragment a wave loads is reused
// across NG weight-row groups; wide layers (N >= 6144 here: >= 192 workgroups
// of 32 columns) take NG = 2 and 8 waves, very wide ones (N >= 16384) NG = 4,
// narrow ones keep one group so every CU still gets a workgroup.
template <int MG>
hipError_t launch_mg_ng(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                        int out_type, int64_t ld_out, hipStream_t s) {
    int ng = decode_ng_knob();
    if (ng == 0) ng = MG == 1 ? 1 : N >= 16384 ? 4 : N >= 6144 ? 2 : 1;
    if (ng == 4) return launch_cfg<MG, 4, 8, 2>(a, w, M, N, K, out, out_type, ld_out, s);
    if (ng == 2) return launch_cfg<MG, 2, 8, 2>(a, w, M, N, K, out, out_type, ld_out, s);
    return launch_mg<MG, 1>(a, w, M, N, K, out, out_type, ld_out, s);
}

hipError_t launch_skinny_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                              int out_type, int64_t ld_out, hipStream_t s) {
    if (M <= 16) return launch_mg_ng<1>(a, w, M, N, K, out, out_type, ld_out, s);
    if (M <= 32) return launch_mg_ng<2>(a, w, M, N, K, out, out_type, ld_out, s);
    if (M <= 64) return launch_mg_ng<4>(a, w, M, N, K, out, out_type, ld_out, s);
    return hipErrorInvalidValue;
}

template <int MG>
hipError_t launch_nv_ng(const uint8_t *ac, const uint8_t *as, const float *aa_in, const uint8_t *wc,
                        const uint8_t *ws, const float *wa, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                        int64_t ld_out, hipStream_t s) {
    float *aa = const_cast<float *>(aa_in);  // only read when A is NVFP4
    int ng = decode_ng_knob();
    // two 16-row weight groups per workgroup on wide layers (each X fragment
    // then serves both): measured faster from N = 6144 at one and four row
    // groups, slower at N = 4096; four groups were slower everywhere
    if (ng == 0) ng = (MG == 1 || MG == 4) && N >= 6144 ? 2 : 1;
    if (MG == 4 && ng == 4) ng = 2;  // four row groups by four column groups exceed the register file
    constexpr int U = MG == 1 ? 2 : 1;  // chunks per register stage
    switch (ng) {
        case 2: return launch_nvfp4_cfg<MG, 2, 8, U>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, s);
        case 4: return launch_nvfp4_cfg<MG, MG == 4 ? 2 : 4, 8, 1>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, s);
        default: return launch_nvfp4_cfg<MG, 1, 16, U>(ac, as, aa, wc, ws, wa, M, N, K, out, out_type, ld_out, s);
    }
}

hipError_t launch_skinny_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                               const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                               int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, hipStream_t s) {
    if (M <= 16)
        return launch_nv_ng<1>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out, s);
    if (M <= 32)
        return launch_nv_ng<2>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out, s);
    if (M <= 64)
        return launch_nv_ng<4>(a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, out, out_type, ld_out, s);
    return hipErrorInvalidValue;
}

hipError_t launch_skinny_fused(const uint16_t *x, int64_t ld_x, float *a_alpha, int dynamic, const uint8_t *w_codes,
                               const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                               void *out, int out_type, int64_t ld_out, hipStream_t s) {
    if (M > 16 || M * K > kFusedDecodeMaxElems) return hipErrorInvalidValue;
    // wide layers: several 16-row weight groups per workgroup, so fewer
    // workgroups quantize the batch (every one of them does)
    const int ng = N >= 16384 ? 4 : N >= 6144 ? 2 : 1;
    if (dynamic) {
        if (ng == 4)
            return launch_nvfp4_cfg<1, 4, 8, 1, A_BF16_DYNAMIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha,
                                                                M, N, K, out, out_type, ld_out, s, x, ld_x);
        if (ng == 2)
            return launch_nvfp4_cfg<1, 2, 8, 1, A_BF16_DYNAMIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha,
                                                                M, N, K, out, out_type, ld_out, s, x, ld_x);
        return launch_nvfp4_cfg<1, 1, 16, 1, A_BF16_DYNAMIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha, M,
                                                             N, K, out, out_type, ld_out, s, x, ld_x);
    }
    if (ng == 4)
        return launch_nvfp4_cfg<1, 4, 8, 1, A_BF16_STATIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha, M, N,
                                                           K, out, out_type, ld_out, s, x, ld_x);
    if (ng == 2)
        return launch_nvfp4_cfg<1, 2, 8, 1, A_BF16_STATIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha, M, N,
                                                           K, out, out_type, ld_out, s, x, ld_x);
    return launch_nvfp4_cfg<1, 1, 16, 1, A_BF16_STATIC>(nullptr, nullptr, a_alpha, w_codes, w_scales, w_alpha, M, N,
                                                        K, out, out_type, ld_out, s, x, ld_x);
}

hipError_t launch_fill_zero(void *out, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t g = rows < 4096 ? rows : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s, (uint8_t *)out, rows, cols * elem_bytes,
                       ld * elem_bytes);
    return hipGetLastError();
}

}  // namespace nvfp4
