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
// 32x32x64).  Interior tiles with K % 512 == 0 run a register-staged
// pipeline with K step 128 and block scales fetched per group of four steps
// (mx_tile_pipe); edge tiles and other K a simpler loop with K step 256, two
// LDS stages of 68 KB staged through guarded register loads (mx_tile_staged).
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
// the K-256 loop of edge tiles
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

// Pipelined interior tiles (K % 512 == 0): K step 128, two LDS stages of A
// and W codes (256 rows x 64 bytes each, swizzled 16-byte chunks), and the
// scales in groups of four steps (16 bytes per row: K 512), two group buffers
// of 8 KB.  Every fragment read is a register base plus an immediate offset.
// Operands are staged through registers from buffer loads: step kt + 2 is
// loaded while step kt computes, and step kt + 1 (loaded one step earlier) is
// written to LDS between the two k64 sub-steps; the step's one barrier
// follows, and the next step's fragments and scales are read under the second
// sub-step's MFMAs.  A row's scales are fetched 16 bytes at a time, once per
// four steps: fetched per step (4 bytes per row), they made half of the L2
// requests of the loop for 6% of its bytes.
constexpr int PKB = 64;                    // code bytes per row per step (128 k)
constexpr int PCODE = MBM * PKB;           // 16 KB
constexpr int PW = 2 * PCODE;              // W code stages
constexpr int PSC = 4 * PCODE;             // scale groups: [2][A 256 x 16 B, W 256 x 16 B]
constexpr int PSG = 2 * MBM * 16;          // 8 KB per group
static_assert(PSC + 2 * PSG <= 2 * STAGE, "the pipelined stages fit the kernel's LDS");

// 16-byte chunk c (of 4) of row r: slot c ^ ((r / 4) % 4), so the 16 rows a
// quarter-wave reads at one chunk fall on distinct banks
__device__ __forceinline__ int pcode_off(int row, int chunk) { return row * PKB + ((chunk ^ ((row >> 2) & 3)) << 4); }

// one step's codes in registers: two 16-byte chunks of A and of W (native
// vectors: HIP's uint4 wrapper kept these in scratch)
struct MxRegs {
    u32x4_t a0, a1, w0, w1;
};

template <bool kOutBf16>
__device__ __forceinline__ void mx_store(const MxArgs &g, const f32x16_t (&acc)[MTM][MTN], int64_t m0, int64_t n0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / MWGN, wn = wave % MWGN;
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

// k64 sub-step ks of a step: 4 x 2 scaled MFMAs; the lane's scale is byte 2 ks
// of its (shifted) scale word
__device__ __forceinline__ void mx_mfmas(f32x16_t (&acc)[MTM][MTN], const uint4 *fa, const uint4 *fb,
                                         const uint32_t *sa, const uint32_t *sw, int ks) {
#pragma unroll
    for (int i = 0; i < MTM; ++i) {
        const i32x8_t a8 = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < MTN; ++j) {
            const i32x8_t b8 = {(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0};
            if (ks)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 2, (int)sa[i], 2,
                                                                            (int)sw[j]);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, (int)sa[i], 0,
                                                                            (int)sw[j]);
        }
    }
}

template <bool kOutBf16>
__device__ __forceinline__ void mx_tile_pipe(const MxArgs &g, uint8_t *smem, int64_t m0, int64_t n0) {
    const int lane = threadIdx.x & 63, t = threadIdx.x;
    const int wave = t >> 6;
    const int wm = wave / MWGN, wn = wave % MWGN;
    const int KT = (int)(g.K / 128);  // a multiple of 4
    const uint32_t rb = (uint32_t)(g.K >> 1), sb = (uint32_t)(g.K >> 5);

    // staging: thread t moves chunks t and t + 512 of each code tile (row
    // i / 4, chunk i % 4) and, once per group, the 16 scale bytes of row t of
    // A (t < 256) or t - 256 of W; buffer resources over the tile's rows, the
    // step as the scalar offset
    const rsrc_t ra_ = make_rsrc(g.ac + m0 * (int64_t)rb, MBM * rb);
    const rsrc_t rw_ = make_rsrc(g.wc + n0 * (int64_t)rb, MBN * rb);
    const int sop = t >> 8, sr = t & 255;
    const rsrc_t rs_ = make_rsrc(sop ? g.ws + n0 * (int64_t)sb : g.as + m0 * (int64_t)sb, MBM * sb);
    uint32_t go[2];
    int lo[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = t + q * 512, r = i >> 2, c = i & 3;
        go[q] = r * rb + c * 16;
        lo[q] = pcode_off(r, c);
    }
    const uint32_t gso = sr * sb;
    const int slo = PSC + sop * (MBM * 16) + sr * 16;
    auto load_regs = [&](MxRegs &R, int kt) __attribute__((always_inline)) {
        const int o = kt * PKB;
        R.a0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra_, go[0], o, 0));
        R.a1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra_, go[1], o, 0));
        R.w0 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw_, go[0], o, 0));
        R.w1 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw_, go[1], o, 0));
    };
    auto store_regs = [&](const MxRegs &R, int b) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4_t *>(smem + b * PCODE + lo[0]) = R.a0;
        *reinterpret_cast<u32x4_t *>(smem + b * PCODE + lo[1]) = R.a1;
        *reinterpret_cast<u32x4_t *>(smem + PW + b * PCODE + lo[0]) = R.w0;
        *reinterpret_cast<u32x4_t *>(smem + PW + b * PCODE + lo[1]) = R.w1;
    };
    auto load_scales = [&](int grp) __attribute__((always_inline)) {
        return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_, gso, grp * 16, 0));
    };
    auto store_scales = [&](u32x4_t v, int gb) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4_t *>(smem + slo + gb * PSG) = v;
    };

    // fragment and scale addresses of this lane: fragment i of A is 32 i rows
    // further (same swizzle), the second k64 sub-step two chunks further
    const int ra = wm * MWM + (lane & 31), rw = wn * MWN + (lane & 31);
    const uint8_t *fa0 = smem + pcode_off(ra, lane >> 5), *fa1 = smem + (pcode_off(ra, lane >> 5) ^ 32);
    const uint8_t *fb0 = smem + PW + pcode_off(rw, lane >> 5), *fb1 = smem + PW + (pcode_off(rw, lane >> 5) ^ 32);
    const uint8_t *sca = smem + PSC + ra * 16, *scw = smem + PSC + MBM * 16 + rw * 16;
    const int sh = 8 * (lane >> 5);  // upper half-wave: the odd 32-block of each k64
    auto read_frags = [&](int b, int ks, uint4 *fa, uint4 *fb) __attribute__((always_inline)) {
        const uint8_t *pa = (ks ? fa1 : fa0) + b * PCODE, *pb = (ks ? fb1 : fb0) + b * PCODE;
#pragma unroll
        for (int i = 0; i < MTM; ++i) fa[i] = *reinterpret_cast<const uint4 *>(pa + i * 32 * PKB);
#pragma unroll
        for (int j = 0; j < MTN; ++j) fb[j] = *reinterpret_cast<const uint4 *>(pb + j * 32 * PKB);
    };
    // step kt's scale words (word kt % 4 of the group's 16 bytes) as stored;
    // shifted for the lane when the step starts, so the reads have a sub-step
    // of MFMAs to land
    auto read_scales = [&](int kt, uint32_t *sa, uint32_t *sw) __attribute__((always_inline)) {
        const int o = ((kt >> 2) & 1) * PSG + (kt & 3) * 4;
#pragma unroll
        for (int i = 0; i < MTM; ++i) sa[i] = *reinterpret_cast<const uint32_t *>(sca + o + i * 32 * 16);
#pragma unroll
        for (int j = 0; j < MTN; ++j) sw[j] = *reinterpret_cast<const uint32_t *>(scw + o + j * 32 * 16);
    };
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); loads stay in flight
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    f32x16_t acc[MTM][MTN];
#pragma unroll
    for (int i = 0; i < MTM; ++i)
#pragma unroll
        for (int j = 0; j < MTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    uint4 fa[2][MTM], fb[2][MTN];
    uint32_t sa[2][MTM], sw[2][MTN];
    MxRegs R0, R1;  // named (not an array), so they stay in registers
    u32x4_t RS;     // the next scale group

    // Every step loads codes two steps ahead (past the end, a repeat of the
    // last step) and stores one step, so the steps are straight-line code;
    // the third step of a group loads the next group's scales, the fourth
    // stores them.
    load_regs(R0, 0);
    store_regs(R0, 0);
    store_scales(load_scales(0), 0);
    load_regs(R1, min(1, KT - 1));
    lds_barrier();
    read_frags(0, 0, fa[0], fb[0]);
    read_scales(0, sa[0], sw[0]);

    // step kt = 4 j + u on code stage b = u % 2 (constants in each unrolled copy)
    auto step = [&](int kt, auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value, b = u & 1;
        uint32_t ssa[MTM], ssw[MTN];
#pragma unroll
        for (int i = 0; i < MTM; ++i) ssa[i] = sa[b][i] >> sh;
#pragma unroll
        for (int j = 0; j < MTN; ++j) ssw[j] = sw[b][j] >> sh;
        // R0 / R1 alternate: the free one loads step kt + 2, the other holds kt + 1
        if constexpr (b == 0)
            load_regs(R0, min(kt + 2, KT - 1));
        else
            load_regs(R1, min(kt + 2, KT - 1));
        if constexpr (u == 2) RS = load_scales(min((kt >> 2) + 1, (KT >> 2) - 1));
        read_frags(b, 1, fa[1], fb[1]);
        // the schedule is kept as written: reads ahead of the MFMAs that
        // cover them, nothing moved across the phases (registers)
        __builtin_amdgcn_sched_barrier(0);
        mx_mfmas(acc, fa[0], fb[0], ssa, ssw, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (b == 0)
            store_regs(R1, 1);
        else
            store_regs(R0, 0);
        if constexpr (u == 3) store_scales(RS, ((kt >> 2) + 1) & 1);
        lds_barrier();
        // (after the last step these read stages nobody uses)
        read_frags(b ^ 1, 0, fa[0], fb[0]);
        read_scales(kt + 1, sa[b ^ 1], sw[b ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        mx_mfmas(acc, fa[1], fb[1], ssa, ssw, 1);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int kt = 0; kt < KT; kt += 4) {
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
        step(kt + 2, std::integral_constant<int, 2>());
        step(kt + 3, std::integral_constant<int, 3>());
    }
    mx_store<kOutBf16>(g, acc, m0, n0);
}

// Edge tiles and K % 512 != 0: K step 256, two LDS stages staged through
// registers; rows past M/N repeat the last row, code chunks past K are zero
// and their scales 1.0 (code 127).
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
__device__ __forceinline__ void mx_tile_staged(const MxArgs &g, uint8_t *smem, int64_t m0, int64_t n0) {
    const int KT = (int)((g.K + 255) / 256);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / MWGN, wn = wave % MWGN;
    auto stage = [&](int s) { return smem + s * STAGE; };

    f32x16_t acc[MTM][MTN];
#pragma unroll
    for (int i = 0; i < MTM; ++i)
#pragma unroll
        for (int j = 0; j < MTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (KT > 0) stage_guarded(g, stage(0), m0, n0, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) stage_guarded(g, stage(cur ^ 1), m0, n0, kt + 1);
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
            uint32_t sai[MTM], swj[MTN];
#pragma unroll
            for (int i = 0; i < MTM; ++i) sai[i] = (ks >> 1) ? sa[i].y : sa[i].x;
#pragma unroll
            for (int j = 0; j < MTN; ++j) swj[j] = (ks >> 1) ? sw[j].y : sw[j].x;
            mx_mfmas(acc, af[ks & 1], bf[ks & 1], sai, swj, ks & 1);
        }
        __syncthreads();
    }
    mx_store<kOutBf16>(g, acc, m0, n0);
}

template <bool kOutBf16>
__global__ __launch_bounds__(MNT, 1) void mx_gemm_kernel(MxArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int tm, tn;
    tile_coords<MBM, MBN>(g.M, g.N, tm, tn);
    const int64_t m0 = (int64_t)tm * MBM, n0 = (int64_t)tn * MBN;
    if (m0 + MBM <= g.M && n0 + MBN <= g.N && (g.K & 511) == 0)
        mx_tile_pipe<kOutBf16>(g, smem, m0, n0);
    else
        mx_tile_staged<kOutBf16>(g, smem, m0, n0);
}

template <bool kOutBf16>
hipError_t launch_mx(const MxArgs &g, hipStream_t s) {
    const int64_t nb = ((g.M + MBM - 1) / MBM) * ((g.N + MBN - 1) / MBN);
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds = 2 * (size_t)STAGE;
    static std::atomic<uint32_t> attr_done{0};
    if (hipError_t e = set_dyn_lds_once(attr_done, (const void *)mx_gemm_kernel<kOutBf16>, (int)lds); e != hipSuccess)
        return e;
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
