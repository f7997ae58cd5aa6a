// MXFP4 for gfx950: E2M1 elements with one E8M0 (power-of-two) scale per 32
// elements along K, the coarser microscaling format Mix-Quant Section 3.3
// contrasts with NVFP4.  Unlike NVFP4's per-16 E4M3 scales, this maps one to
// one onto the block-scaled FP4 MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 takes
// 32 packed FP4 values and one E8M0 scale per lane, i.e. per (row, 32-block).
//
// Quantizer (OCP MX v1.0 conversion): shared exponent floor(log2 amax) - 2,
// clamped to [-127, 127] (-127 for an all-zero block); each element scaled by
// 2^-shared (exact) and rounded to E2M1 nearest-even with saturation by the
// hardware FP32 -> FP4 convert.  Four lanes of 8 elements share a block and
// combine their maxima with two DPP swaps.
//
// GEMM: 256 x 256 output tile, 8 waves of 128 x 64 (4 x 2 scaled MFMAs of
// 32x32x64), K step 256 (128 bytes of codes per row, the same LDS row shape
// and swizzle as the FP16 GEMM), two LDS stages of 68 KB.  Interior steps
// are staged with direct global -> LDS loads (global_load_lds_dwordx4: no
// registers, no ALU; scales 4 bytes per lane); row and K tails with guarded
// register loads.
#include <stdlib.h>
#include <string.h>

#include "internal.hpp"
#include "nvfp4_device.hpp"
#include "tiling.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// ------------------------------------------------------------------ quantize
constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;

__global__ __launch_bounds__(kQThreads) void mx_quantize_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ld, uint8_t *__restrict__ codes,
                                                                uint8_t *__restrict__ scales) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t octs = cols >> 3;  // multiple of 4: a block's four lanes never straddle rows
    constexpr int U = 4;
    for (int64_t r = (int64_t)blockIdx.x * kQWaves + wave; r < rows; r += (int64_t)gridDim.x * kQWaves) {
        const uint4 *xr = reinterpret_cast<const uint4 *>(x + r * ld);
        uint32_t *cr = reinterpret_cast<uint32_t *>(codes + r * (cols >> 1));
        uint8_t *sr = scales + r * (cols >> 5);
        for (int64_t o0 = lane; o0 < octs; o0 += 64 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = (o0 + 64 * u < octs) ? load_nt16(xr + o0 + 64 * u) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = o0 + 64 * u;
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                uint32_t am = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
                am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false));  // lane ^ 1
                am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0x4E, 0xF, 0xF, false));  // lane ^ 2
                const float amax = bf16_bits_to_f32(am);
                int shared = -127;
                if (amax > 0.0f) shared = min(127, max(-127, __builtin_amdgcn_frexp_expf(amax) - 1 - 2));
                float a[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[2 * i] = __builtin_ldexpf(bf16_bits_to_f32(w[i] & 0xFFFFu), -shared);
                    a[2 * i + 1] = __builtin_ldexpf(bf16_bits_to_f32(w[i] >> 16), -shared);
                }
                uint32_t packed = 0;
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[0], a[1], 1.0f, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[2], a[3], 1.0f, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[4], a[5], 1.0f, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[6], a[7], 1.0f, 3);
                if (o < octs) {
                    cr[o] = packed;
                    if ((o & 3) == 0) sr[o >> 2] = (uint8_t)(shared + 127);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------- GEMM
constexpr int MBM = 256, MBN = 256, MNT = 512;
constexpr int MWGN = 4;                // waves along N (2 along M)
constexpr int MWM = 128, MWN = 64;     // wave tile
constexpr int MTM = MWM / 32, MTN = MWN / 32;
constexpr int MKB = 128;               // code bytes per row per step (256 k)
constexpr int MKS = MKB / 32;          // 32x32x64 MFMA k-substeps per step
constexpr int CODE_TILE = MBM * MKB;   // 32 KB
constexpr int SCALE_TILE = MBM * 8;    // 2 KB (8 E8M0 scales per row per step)
constexpr int STAGE = 2 * CODE_TILE + 2 * SCALE_TILE;
static_assert(MBM == MBN, "square tiles");

struct MxArgs {
    const uint8_t *ac, *as, *wc, *ws;
    int64_t M, N, K;
    void *out;
    int64_t ld_out;
};

__device__ __forceinline__ int code_off(int row, int chunk) { return row * MKB + ((chunk ^ lds_swz(row)) << 4); }

// Direct global -> LDS staging of one step (interior rows, whole step in K).
// Code tiles: each wave instruction fills 1 KB = 8 rows; lane l writes slot
// l % 8 of row l / 8, so it fetches logical chunk slot ^ f(row).
__device__ __forceinline__ void stage_direct(const MxArgs &g, uint8_t *stage, int64_t m0, int64_t n0, int kt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rb = g.K >> 1, sb = g.K >> 5;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
        const uint8_t *src = op ? g.wc : g.ac;
        const int64_t row0 = op ? n0 : m0;
        uint8_t *dst = stage + op * CODE_TILE;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int base = wave * 32 + q * 8;  // first tile row of this instruction
            const int r = base + (lane >> 3), slot = lane & 7;
            const int chunk = slot ^ lds_swz(r);
            const uint8_t *gp = src + (row0 + r) * rb + (int64_t)kt * MKB + chunk * 16;
            __builtin_amdgcn_global_load_lds(gp, dst + base * MKB, 16, 0, 0);
        }
    }
    // scales: 8 bytes per row = two dwords; waves 0-3 stage A's 512 dwords,
    // waves 4-7 W's, 64 dwords (32 rows) per instruction
    {
        const int op = wave >> 2;
        const uint8_t *src = op ? g.ws : g.as;
        const int64_t row0 = op ? n0 : m0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int base = (wave & 3) * 128 + q * 64;  // first dword of this instruction
            const int idx = base + lane, r = idx >> 1;
            const uint8_t *gp = src + (row0 + r) * sb + (int64_t)kt * 8 + (idx & 1) * 4;
            __builtin_amdgcn_global_load_lds(gp, stage + 2 * CODE_TILE + op * SCALE_TILE + base * 4, 4, 0, 0);
        }
    }
}

// Guarded staging through registers: rows past M/N repeat the last row, code
// chunks past K are zero and their scales 1.0 (code 127).
__device__ __forceinline__ void stage_guarded(const MxArgs &g, uint8_t *stage, int64_t m0, int64_t n0, int kt) {
    const int64_t rb = g.K >> 1, sb = g.K >> 5;
#pragma unroll
    for (int op = 0; op < 2; ++op) {
        const uint8_t *src = op ? g.wc : g.ac;
        const int64_t row0 = op ? n0 : m0, rows = op ? g.N : g.M;
        uint8_t *dst = stage + op * CODE_TILE;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = threadIdx.x + q * MNT;  // chunk index in the tile
            const int r = i >> 3, c = i & 7;
            const int64_t grow = min(row0 + r, rows - 1);
            const int64_t kbyte = (int64_t)kt * MKB + c * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (kbyte + 16 <= rb) v = *reinterpret_cast<const uint4 *>(src + grow * rb + kbyte);
            *reinterpret_cast<uint4 *>(dst + code_off(r, c)) = v;
        }
    }
    if (threadIdx.x < 2 * MBM) {
        const int op = threadIdx.x >= MBM, r = threadIdx.x & (MBM - 1);
        const uint8_t *src = op ? g.ws : g.as;
        const int64_t row0 = op ? n0 : m0, rows = op ? g.N : g.M;
        const int64_t grow = min(row0 + r, rows - 1);
        uint8_t s8[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int64_t blk = (int64_t)kt * 8 + b;
            s8[b] = blk < sb ? src[grow * sb + blk] : (uint8_t)127;
        }
        uint8_t *dst = stage + 2 * CODE_TILE + op * SCALE_TILE + r * 8;
        *reinterpret_cast<u32x2_t *>(dst) =
            u32x2_t{(uint32_t)s8[0] | ((uint32_t)s8[1] << 8) | ((uint32_t)s8[2] << 16) | ((uint32_t)s8[3] << 24),
                    (uint32_t)s8[4] | ((uint32_t)s8[5] << 8) | ((uint32_t)s8[6] << 16) | ((uint32_t)s8[7] << 24)};
    }
}

template <bool kOutBf16>
__global__ __launch_bounds__(MNT, 1) void mx_gemm_kernel(MxArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int tm, tn;
    tile_coords<MBM, MBN>(g.M, g.N, tm, tn);
    const int64_t m0 = (int64_t)tm * MBM, n0 = (int64_t)tn * MBN;
    const int KT = (int)((g.K + 255) / 256);
    const bool direct = m0 + MBM <= g.M && n0 + MBN <= g.N && (g.K & 255) == 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / MWGN, wn = wave % MWGN;
    auto stage = [&](int s) { return smem + s * STAGE; };
    auto fill = [&](int s, int kt) __attribute__((always_inline)) {
        if (direct)
            stage_direct(g, stage(s), m0, n0, kt);
        else
            stage_guarded(g, stage(s), m0, n0, kt);
    };

    f32x16_t acc[MTM][MTN];
#pragma unroll
    for (int i = 0; i < MTM; ++i)
#pragma unroll
        for (int j = 0; j < MTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (KT > 0) fill(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) fill(cur ^ 1, kt + 1);
        const uint8_t *A = stage(cur), *W = stage(cur) + CODE_TILE;
        const uint8_t *SA = stage(cur) + 2 * CODE_TILE, *SW = SA + SCALE_TILE;
        // per fragment row: the step's 8 E8M0 scales, shifted so that byte
        // 2(j & 1) of word j >> 1 is the lane's block (2j for lanes 0-31,
        // 2j + 1 for lanes 32-63)
        u32x2_t sa[MTM], sw[MTN];
        const int sh = 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < MTM; ++i) {
            sa[i] = *reinterpret_cast<const u32x2_t *>(SA + (wm * MWM + i * 32 + (lane & 31)) * 8);
            sa[i] = u32x2_t{sa[i].x >> sh, sa[i].y >> sh};
        }
#pragma unroll
        for (int j = 0; j < MTN; ++j) {
            sw[j] = *reinterpret_cast<const u32x2_t *>(SW + (wn * MWN + j * 32 + (lane & 31)) * 8);
            sw[j] = u32x2_t{sw[j].x >> sh, sw[j].y >> sh};
        }
        uint4 af[2][MTM], bf[2][MTN];
        auto read_frags = [&](int ks, uint4 *fa, uint4 *fb) __attribute__((always_inline)) {
            const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
            for (int i = 0; i < MTM; ++i)
                fa[i] = *reinterpret_cast<const uint4 *>(A + code_off(wm * MWM + i * 32 + (lane & 31), chunk));
#pragma unroll
            for (int j = 0; j < MTN; ++j)
                fb[j] = *reinterpret_cast<const uint4 *>(W + code_off(wn * MWN + j * 32 + (lane & 31), chunk));
        };
        read_frags(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < MKS; ++ks) {
            if (ks + 1 < MKS) read_frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < MTM; ++i) {
                const uint4 a = af[ks & 1][i];
                const i32x8_t a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                const int sai = (int)((ks >> 1) ? sa[i].y : sa[i].x);
#pragma unroll
                for (int j = 0; j < MTN; ++j) {
                    const uint4 b = bf[ks & 1][j];
                    const i32x8_t b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
                    const int swj = (int)((ks >> 1) ? sw[j].y : sw[j].x);
                    if (ks & 1)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 2, sai,
                                                                                    2, swj);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, sai,
                                                                                    0, swj);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the next stage (direct loads) has landed
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < MTM; ++i)
#pragma unroll
        for (int j = 0; j < MTN; ++j) {
            const int64_t col = n0 + wn * MWN + j * 32 + (lane & 31);
            if (col >= g.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * MWM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row >= g.M) continue;
                if (kOutBf16)
                    reinterpret_cast<__bf16 *>(g.out)[row * g.ld_out + col] = (__bf16)acc[i][j][r];
                else
                    reinterpret_cast<float *>(g.out)[row * g.ld_out + col] = acc[i][j][r];
            }
        }
}

template <bool kOutBf16>
hipError_t launch_mx(const MxArgs &g, hipStream_t s) {
    const int64_t nb = ((g.M + MBM - 1) / MBM) * ((g.N + MBN - 1) / MBN);
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)STAGE;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)mx_gemm_kernel<kOutBf16>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(mx_gemm_kernel<kOutBf16>, dim3((unsigned)nb), dim3(MNT), lds, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                              uint8_t *scales, hipStream_t s) {
    int64_t grid = (rows + kQWaves - 1) / kQWaves;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, s, x, rows, cols, ld, codes,
                       scales);
    return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                          const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                          int64_t ld_out, hipStream_t s) {
    MxArgs g{a_codes, a_scales, w_codes, w_scales, M, N, K, out, ld_out};
    return out_type == OUT_BF16 ? launch_mx<true>(g, s) : launch_mx<false>(g, s);
}

}  // namespace nvfp4
