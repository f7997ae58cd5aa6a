// Tile GEMMs for gfx950: Y[M, N] = A[M, K] * W[N, K]^T with FP32 accumulation.
//
// NVFP4 x NVFP4 (Mix-Quant Section 3.3, Eq. 2; W4A4 prefill linears of
// Section 4.2).  gfx950's block-scaled FP4 MFMAs apply one power-of-two
// (E8M0) scale per 32 K-elements, while NVFP4 carries an arbitrary E4M3
// scale per 16 K-elements on both operands; the per-block factor
// sigmaA[m,b] * sigmaW[n,b] cannot be taken out of the hardware K-sum, and
// re-encoding q * sigma (up to 6 significant bits) in FP8/FP6 loses bits.
// So each operand tile is expanded once per workgroup, while it is staged
// into LDS, to FP16 values q * sigma -- exact, since q has 2 and sigma 4
// significant bits and both lie well inside FP16's range -- and the main
// loop runs FP16 MFMAs.  The tensor scales alphaA * alphaW are applied in
// the epilogue.  The same main loop serves the BF16 GEMM (BF16 MFMAs on
// copied tiles) and the fused path that quantizes BF16 activations in the
// staging step.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of
// 64 x 64, each a 2 x 2 grid of 32x32x16 MFMAs), K step 64, LDS double
// buffer (64 KB).  LDS rows are 64 halves = eight 16-byte chunks; chunk c of
// row r lives at chunk slot c ^ (r & 7) so the MFMA operand reads (8 rows x
// 16 bytes per lane octet) hit all 32 banks once.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NT = 256;
constexpr int TILE = BM * BK;  // 16-bit elements per operand tile (BM == BN)
static_assert(BM == BN, "loaders assume square tiles");

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

struct GemmArgs {
    const void *a;          // A codes, A BF16
    const uint8_t *a_scales;
    const float *a_alpha;
    const void *w;          // W codes or W BF16
    const uint8_t *w_scales;
    const float *w_alpha;
    int64_t M, N, K, lda;   // lda: BF16 row stride (fused / BF16 A)
    void *out;
    int64_t ld_out;
};

// ---------------------------------------------------------------- loaders
// Every loader moves one [128 rows x 64 k] operand tile: thread t owns row
// t >> 1 and k-half (t & 1) * 32 .. +32, i.e. two NVFP4 blocks.

struct Fp4Stage {
    uint4 codes;
    uint32_t sc;  // two scale bytes
};

__device__ __forceinline__ void fp4_load(Fp4Stage &st, const uint8_t *__restrict__ codes,
                                         const uint8_t *__restrict__ scales, int64_t rows, int64_t K,
                                         int64_t row0, int kt) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const int64_t row = row0 + r;
    const int64_t k0 = (int64_t)kt * BK + h * 32;
    st.codes = make_uint4(0, 0, 0, 0);
    st.sc = 0;
    if (row < rows) {
        const uint8_t *cp = codes + row * (K >> 1) + (k0 >> 1);
        const uint8_t *sp = scales + row * (K >> 4) + (k0 >> 4);
        if (k0 + 32 <= K) {
            if ((K & 31) == 0) {
                st.codes = *reinterpret_cast<const uint4 *>(cp);
            } else {
                uint2 lo = *reinterpret_cast<const uint2 *>(cp), hi = *reinterpret_cast<const uint2 *>(cp + 8);
                st.codes = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            st.sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
        } else if (k0 + 16 <= K) {
            uint2 lo = *reinterpret_cast<const uint2 *>(cp);
            st.codes = make_uint4(lo.x, lo.y, 0, 0);
            st.sc = sp[0];
        }
    }
}

// 8 E2M1 codes (one 32-bit word) times sigma -> 8 FP16 values (exact).
__device__ __forceinline__ half8_t expand8(uint32_t w, half_t sigma) {
    half8_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint16_t b = (uint16_t)e2m1_to_f16_bits((w >> (4 * i)) & 15u);
        v[i] = __builtin_bit_cast(half_t, b) * sigma;
    }
    return v;
}

__device__ __forceinline__ void fp4_store(const Fp4Stage &st, half_t *lds) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const half_t s0 = e4m3_to_f16(st.sc & 0xFFu), s1 = e4m3_to_f16(st.sc >> 8);
    const uint32_t w[4] = {st.codes.x, st.codes.y, st.codes.z, st.codes.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
        *reinterpret_cast<half8_t *>(lds + lds_off(r, h * 4 + c)) = expand8(w[c], c < 2 ? s0 : s1);
}

struct Bf16Stage {
    uint4 v[4];  // 32 BF16 values
};

__device__ __forceinline__ void bf16_load(Bf16Stage &st, const uint16_t *__restrict__ x, int64_t ld, int64_t rows,
                                          int64_t K, int64_t row0, int kt) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const int64_t row = row0 + r;
    const int64_t k0 = (int64_t)kt * BK + h * 32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        st.v[c] = make_uint4(0, 0, 0, 0);
        if (row < rows && k0 + 8 * c + 8 <= K)
            st.v[c] = *reinterpret_cast<const uint4 *>(x + row * ld + k0 + 8 * c);
    }
}

__device__ __forceinline__ void bf16_store(const Bf16Stage &st, uint16_t *lds) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4 *>(lds + lds_off(r, h * 4 + c)) = st.v[c];
}

// Fused prologue: quantize the staged BF16 values exactly as the standalone
// quantizer does (same block_scale / quant_elem), then expand q * sigma.
__device__ __forceinline__ void fused_store(const Bf16Stage &st, half_t *lds, float alpha) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const uint32_t w[8] = {st.v[2 * b].x, st.v[2 * b].y, st.v[2 * b].z, st.v[2 * b].w,
                               st.v[2 * b + 1].x, st.v[2 * b + 1].y, st.v[2 * b + 1].z, st.v[2 * b + 1].w};
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
        const BlockScale bs = block_scale(bf16_bits_to_f32(am), alpha);
        const half_t sig = (half_t)bs.sigma;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t x = w[4 * c + i];
                packed |= quant_elem(bf16_bits_to_f32(x & 0xFFFFu), bs.d) << (8 * i);
                packed |= quant_elem(bf16_bits_to_f32(x >> 16), bs.d) << (8 * i + 4);
            }
            *reinterpret_cast<half8_t *>(lds + lds_off(r, h * 4 + 2 * b + c)) = expand8(packed, sig);
        }
    }
}

// ---------------------------------------------------------------- kernel
enum Kind { KIND_NVFP4 = 0, KIND_FUSED = 1, KIND_BF16 = 2 };

__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int &tm, int &tn) {
    const int num_tm = (int)((M + BM - 1) / BM), num_tn = (int)((N + BN - 1) / BN);
    const int nb = gridDim.x;
    int bid = blockIdx.x;
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous range of logical tiles so neighbouring tiles share its L2.
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    constexpr int G = 8;  // tiles along M per group: W tiles are reused across it
    const int per_group = G * num_tn;
    const int group = bid / per_group;
    const int first_tm = group * G;
    const int gsize = min(num_tm - first_tm, G);
    const int in = bid % per_group;
    tm = first_tm + in % gsize;
    tn = in / gsize;
}

template <int kKind, bool kOutBf16>
__global__ __launch_bounds__(NT, 2) void gemm_kernel(GemmArgs g) {
    typedef typename std::conditional<kKind == KIND_BF16, uint16_t, half_t>::type lds_t;
    __shared__ __attribute__((aligned(16))) lds_t lds[2][2][TILE];

    int tm, tn;
    tile_coords(g.M, g.N, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int KT = (int)((g.K + BK - 1) / BK);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    float a_alpha = 1.0f;
    if (kKind == KIND_FUSED) a_alpha = *g.a_alpha;

    Fp4Stage sa4, sw4;
    Bf16Stage sab, swb;

    auto load = [&](int kt) {
        if (kKind == KIND_NVFP4)
            fp4_load(sa4, (const uint8_t *)g.a, g.a_scales, g.M, g.K, m0, kt);
        else
            bf16_load(sab, (const uint16_t *)g.a, g.lda, g.M, g.K, m0, kt);
        if (kKind == KIND_BF16)
            bf16_load(swb, (const uint16_t *)g.w, g.K, g.N, g.K, n0, kt);
        else
            fp4_load(sw4, (const uint8_t *)g.w, g.w_scales, g.N, g.K, n0, kt);
    };
    auto store = [&](int buf) {
        if (kKind == KIND_NVFP4) fp4_store(sa4, (half_t *)lds[buf][0]);
        if (kKind == KIND_FUSED) fused_store(sab, (half_t *)lds[buf][0], a_alpha);
        if (kKind == KIND_BF16) bf16_store(sab, (uint16_t *)lds[buf][0]);
        if (kKind == KIND_BF16)
            bf16_store(swb, (uint16_t *)lds[buf][1]);
        else
            fp4_store(sw4, (half_t *)lds[buf][1]);
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (KT > 0) {
        load(0);
        store(0);
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load(kt + 1);
        const lds_t *As = lds[cur][0];
        const lds_t *Ws = lds[cur][1];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int chunk = 2 * ks + (lane >> 5);
            uint4 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const uint4 *>(As + lds_off(ra, chunk));
                const int rb = wn * 64 + i * 32 + (lane & 31);
                bf[i] = *reinterpret_cast<const uint4 *>(Ws + lds_off(rb, chunk));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (kKind == KIND_BF16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                                            __builtin_bit_cast(bf16x8_t, bf[j]),
                                                                            acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, af[i]),
                                                                           __builtin_bit_cast(half8_t, bf[j]),
                                                                           acc[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < KT) store(cur ^ 1);
        __syncthreads();
    }

    // epilogue: y = (acc * alphaA) * alphaW, stored FP32 or BF16 (nearest-even)
    float sa = 1.0f, sw = 1.0f;
    if (kKind != KIND_BF16) {
        sa = *g.a_alpha;
        sw = *g.w_alpha;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row >= g.M) continue;
                float y = acc[i][j][r];
                if (kKind != KIND_BF16) y = (y * sa) * sw;
                if (kOutBf16)
                    reinterpret_cast<uint16_t *>(g.out)[row * g.ld_out + col] = (uint16_t)f32_to_bf16_bits(y);
                else
                    reinterpret_cast<float *>(g.out)[row * g.ld_out + col] = y;
            }
        }
}

template <int kKind>
hipError_t launch(const GemmArgs &g, int out_type, hipStream_t s) {
    const int64_t num_tm = (g.M + BM - 1) / BM, num_tn = (g.N + BN - 1) / BN;
    const int64_t nb = num_tm * num_tn;
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (out_type == OUT_BF16)
        hipLaunchKernelGGL((gemm_kernel<kKind, true>), dim3((unsigned)nb), dim3(NT), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_kernel<kKind, false>), dim3((unsigned)nb), dim3(NT), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                             int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, 0, out, ld_out};
    return launch<KIND_NVFP4>(g, out_type, s);
}

hipError_t launch_gemm_fused(const uint16_t *x, int64_t ld_x, const float *a_alpha, const uint8_t *w_codes,
                             const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                             void *out, int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{x, nullptr, a_alpha, w_codes, w_scales, w_alpha, M, N, K, ld_x, out, ld_out};
    return launch<KIND_FUSED>(g, out_type, s);
}

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                            int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{a, nullptr, nullptr, w, nullptr, nullptr, M, N, K, K, out, ld_out};
    return launch<KIND_BF16>(g, out_type, s);
}

}  // namespace nvfp4
