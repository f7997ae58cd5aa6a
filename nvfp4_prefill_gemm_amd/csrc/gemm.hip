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
// Tiling (TileCfg): large problems use a 256 x 256 output tile per
// 512-thread workgroup, 2 x 4 waves of 128 x 64 (a 4 x 2 grid of 32x32x16
// MFMAs each, 128 FP32 accumulators per lane; two waves per SIMD, so one
// wave's staging work overlaps the other's MFMAs), K step 64 and a double-
// buffered LDS stage of 2 x 64 KB; the fused prologue a 256 x 256 tile of
// 4 waves of 128 x 128 (its registers do not fit beside 8 waves); small
// problems a 128 x 128 tile of 4 waves of 64 x 64.  Operand fragments are read from LDS one k16 step ahead
// of the MFMAs that use them; the next K step's global loads are issued
// before the current step's MFMAs (through buffer resources: see the
// loaders).  LDS rows are 64 halves = eight 16-byte
// chunks, swizzled (lds_off) so operand reads and staging writes are free of
// bank conflicts.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include <utility>

#include "internal.hpp"
#include "nvfp4_device.hpp"
#include "epilogue.hpp"
#include "tiling.hpp"

namespace nvfp4 {

namespace {

constexpr int BK = 64;  // K elements per pipeline step (four NVFP4 blocks)

template <int BM_, int BN_, int WGM_, int WGN_, int MINB_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, MINB = MINB_;
    static constexpr int NT = WGM * WGN * 64;
    static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    static constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 MFMA tiles per wave
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
};
using BigTile = TileCfg<256, 256, 2, 2, 1>;   // 4 waves of 128 x 128
using BigTile8 = TileCfg<256, 256, 2, 4, 1>;  // 8 waves of 128 x 64
using SmallTile = TileCfg<128, 128, 2, 2, 2>; // 4 waves of 64 x 64

// LDS tile layout: rows of 64 halves (eight 16-byte chunks), swizzled by lds_swz.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ lds_swz(row)) << 3); }

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled
// by construction (array indices inside f are compile-time constants).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

struct GemmArgs {
    const void *a;          // A codes or A BF16
    const uint8_t *a_scales;
    const float *a_alpha;
    const void *w;          // W codes or W BF16
    const uint8_t *w_scales;
    const float *w_alpha;
    int64_t M, N, K, lda;   // lda: BF16 row stride (fused / BF16 A)
    void *out;
    int64_t ld_out;
    uint8_t *out_scales;      // NVFP4 output: E4M3 block scales [M, N/16]
    const float *out_alpha;   // NVFP4 output: static tensor scale
    uint32_t *amax_part = nullptr;  // OUT_F32_AMAX: 8 slots per workgroup
    int rows_rsrc = 0;        // edge tiles may address a tile's rows through one buffer resource (< 2^31 bytes)
    bool vec = false;         // FP32/BF16 output: out and ld_out allow 16-byte stores
};

// ---------------------------------------------------------------- loaders
// A loader moves one [R rows x 64 k] operand tile with NT threads; each thread
// owns EPT = R * 64 / NT consecutive k of one row (32 or 64: two or four
// NVFP4 blocks).

template <int R, int NT>
struct Part {
    static constexpr int EPT = R * BK / NT;
    static constexpr int PER_ROW = BK / EPT;
    static_assert(EPT == 32 || EPT == 64, "unsupported loader split");
    __device__ __forceinline__ static int row() { return threadIdx.x / PER_ROW; }
    __device__ __forceinline__ static int part() { return threadIdx.x % PER_ROW; }
};

template <int EPT>
struct Fp4Stage {
    uint4 codes[EPT / 32];
    uint32_t sc;  // EPT/16 scale bytes
};

// Operand loads per tile mode.  0 and 1 (K % 64 == 0, a tile's rows fit one
// buffer resource): loads through a buffer resource over the tile's valid
// rows, so rows past the matrix edge (mode 1) read zeros without branches;
// buffer loads with 32-bit offsets also measured faster than global loads on
// interior tiles (mode 0).  4: as 0, the scales supplied by the caller.
// 3: interior tile with plain global loads (the fused kind, measured faster
// that way).  2: any tail, per-access checks.
template <int R, int NT, int kMode>
__device__ __forceinline__ void fp4_load(Fp4Stage<Part<R, NT>::EPT> &st, const uint8_t *__restrict__ codes,
                                         const uint8_t *__restrict__ scales, int64_t rows, int64_t K, int64_t row0,
                                         int kt) {
    constexpr int EPT = Part<R, NT>::EPT;
    const int64_t row = row0 + Part<R, NT>::row();
    const int64_t k0 = (int64_t)kt * BK + Part<R, NT>::part() * EPT;
    if (kMode <= 1 || kMode == 4) {  // 4: the scales come from the caller's per-group loads
        const int64_t nrows = rows - row0 < R ? rows - row0 : R;
        const rsrc_t cs = make_rsrc(codes + row0 * (K >> 1), (uint32_t)(nrows * (K >> 1)));
        const uint32_t rr = (uint32_t)Part<R, NT>::row();
        const uint32_t co = rr * (uint32_t)(K >> 1) + (uint32_t)(k0 >> 1);
#pragma unroll
        for (int i = 0; i < EPT / 32; ++i) st.codes[i] = buf_load16(cs, co + 16 * i);
        if constexpr (kMode != 4) {
            const rsrc_t ss = make_rsrc(scales + row0 * (K >> 4), (uint32_t)(nrows * (K >> 4)));
            const uint32_t so = rr * (uint32_t)(K >> 4) + (uint32_t)(k0 >> 4);
            st.sc = EPT == 64 ? buf_load4(ss, so) : buf_load2(ss, so);
        }
        return;
    }
    if (kMode == 3) {  // interior tile, K % 64 == 0: every access is in range
        const uint8_t *cp = codes + row * (K >> 1) + (k0 >> 1);
#pragma unroll
        for (int i = 0; i < EPT / 32; ++i) st.codes[i] = *reinterpret_cast<const uint4 *>(cp + 16 * i);
        const uint8_t *sp = scales + row * (K >> 4) + (k0 >> 4);
        st.sc = EPT == 64 ? *reinterpret_cast<const uint32_t *>(sp) : *reinterpret_cast<const uint16_t *>(sp);
        return;
    }
#pragma unroll
    for (int i = 0; i < EPT / 32; ++i) st.codes[i] = make_uint4(0, 0, 0, 0);
    st.sc = 0;
    if (row >= rows) return;
    const uint8_t *cp = codes + row * (K >> 1) + (k0 >> 1);
    const uint8_t *sp = scales + row * (K >> 4) + (k0 >> 4);
    if (k0 + EPT <= K && (K & 63) == 0) {
        // whole chunk in range; 16-byte code loads and one aligned scale word
#pragma unroll
        for (int i = 0; i < EPT / 32; ++i) st.codes[i] = *reinterpret_cast<const uint4 *>(cp + 16 * i);
        if (EPT == 64)
            st.sc = *reinterpret_cast<const uint32_t *>(sp);
        else
            st.sc = *reinterpret_cast<const uint16_t *>(sp);
        return;
    }
#pragma unroll
    for (int b = 0; b < EPT / 16; ++b) {  // block by block, 8 code bytes each
        if (k0 + 16 * b + 16 <= K) {
            const uint2 c = *reinterpret_cast<const uint2 *>(cp + 8 * b);
            if (b & 1) {
                st.codes[b >> 1].z = c.x;
                st.codes[b >> 1].w = c.y;
            } else {
                st.codes[b >> 1].x = c.x;
                st.codes[b >> 1].y = c.y;
            }
            st.sc |= (uint32_t)sp[b] << (8 * b);
        }
    }
}

// H selects which half of the thread's blocks to stage (-1: all of them)
template <int R, int NT, int H = -1>
__device__ __forceinline__ void fp4_store(const Fp4Stage<Part<R, NT>::EPT> &st, half_t *lds) {
    constexpr int EPT = Part<R, NT>::EPT;
    constexpr int NB = EPT / 16, B0 = H < 0 ? 0 : H * NB / 2, B1 = H < 0 ? NB : (H + 1) * NB / 2;
    const int r = Part<R, NT>::row(), c0 = Part<R, NT>::part() * (EPT / 8);
#pragma unroll
    for (int b = B0; b < B1; ++b) {
        const half2_t s2 = e4m3_to_f16x2_over256((st.sc >> (8 * b)) & 0xFFu);
        const uint4 &q = st.codes[b >> 1];
        const uint32_t w0 = (b & 1) ? q.z : q.x, w1 = (b & 1) ? q.w : q.y;
        *reinterpret_cast<half8_t *>(lds + lds_off(r, c0 + 2 * b)) = expand8(w0, s2);
        *reinterpret_cast<half8_t *>(lds + lds_off(r, c0 + 2 * b + 1)) = expand8(w1, s2);
    }
}

template <int EPT>
struct Bf16Stage {
    u32x4_t v[EPT / 8];
};


// BF16 operands (BF16 kind, and A of the fused kind), row-interleaved: load c
// of thread t is 16-byte chunk (t + NT c) % 8 of tile row (t + NT c) / 8, so
// each wave instruction reads 8 whole 128-byte row segments (8 L2 requests);
// a thread per row read one 16-byte piece of 64 rows per instruction (64
// requests), 5% slower for the BF16 GEMM at 8192 tokens, 12% at 512.
template <int R, int NT, int kMode>
__device__ __forceinline__ void bf16_load(Bf16Stage<Part<R, NT>::EPT> &st, const uint16_t *__restrict__ x,
                                             int64_t ld, int64_t rows, int64_t K, int64_t row0, int kt) {
    constexpr int EPT = Part<R, NT>::EPT;
    static_assert(BK == 64, "8 chunks per row and step");
    if (kMode <= 1) {  // buffer resource over the valid rows (see fp4_load)
        const int64_t nrows = rows - row0 < R ? rows - row0 : R;
        const rsrc_t xs = make_rsrc(x + row0 * ld, (uint32_t)(nrows * ld * 2));
#pragma unroll
        for (int c = 0; c < EPT / 8; ++c) {
            const uint32_t id = threadIdx.x + NT * c;
            const uint32_t xo = ((id >> 3) * (uint32_t)ld + (uint32_t)kt * BK + (id & 7) * 8) * 2u;
            st.v[c] = __builtin_bit_cast(u32x4_t, buf_load16(xs, xo));
        }
        return;
    }
#pragma unroll
    for (int c = 0; c < EPT / 8; ++c) {
        const int id = threadIdx.x + NT * c;
        const int64_t row = row0 + (id >> 3), k = (int64_t)kt * BK + (id & 7) * 8;
        st.v[c] = (kMode == 3 || (row < rows && k + 8 <= K)) ? *reinterpret_cast<const u32x4_t *>(x + row * ld + k)
                                                            : u32x4_t{0, 0, 0, 0};
    }
}

template <int R, int NT, int H = -1>
__device__ __forceinline__ void bf16_store(const Bf16Stage<Part<R, NT>::EPT> &st, uint16_t *lds) {
    constexpr int EPT = Part<R, NT>::EPT;
    constexpr int NC = EPT / 8, C0 = H < 0 ? 0 : H * NC / 2, C1 = H < 0 ? NC : (H + 1) * NC / 2;
#pragma unroll
    for (int c = C0; c < C1; ++c) {
        const int id = threadIdx.x + NT * c;
        *reinterpret_cast<u32x4_t *>(lds + lds_off(id >> 3, id & 7)) = st.v[c];
    }
}


// Per-workgroup constants of the fused prologue: the tensor scale, Eq. 3's
// t = alpha * 6 with rt = RN(1/t) and the range where the corrected quotient
// amax / t is exact, and per E4M3 code c the divisor d = alpha * sigma(c),
// RN(1/d) and the largest amax the fast Eq. 2 path takes (-1 when d is
// outside [2^-90, 2^100]).
struct FusedQuant {
    float alpha, t, rt, tlim;
    bool tfast;
    const float4 *dtab;
};


// Fused prologue: quantize the staged BF16 values with the standalone
// quantizer's arithmetic (Eq. 3 by the corrected quotient against t, else the
// IEEE quotient; Eq. 2 by quant8_fast, or quant8 for a block outside its
// range), then expand q * sigma.  A lane holds half a block (8 elements, the
// row-interleaved staging above); the block amax takes the partner lane's
// half by one DPP swap, both lanes form the block's scale, and each
// quantizes its own 8 elements.
template <int R, int NT, int H = -1>
__device__ __forceinline__ void fused_store(const Bf16Stage<Part<R, NT>::EPT> &st, half_t *lds,
                                               const FusedQuant &fq) {
    constexpr int EPT = Part<R, NT>::EPT;
    constexpr int NC = EPT / 8, C0 = H < 0 ? 0 : H * NC / 2, C1 = H < 0 ? NC : (H + 1) * NC / 2;
#pragma unroll
    for (int c = C0; c < C1; ++c) {
        const int id = threadIdx.x + NT * c;
        const uint32_t w[4] = {st.v[c].x, st.v[c].y, st.v[c].z, st.v[c].w};
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w[i] << 16)),
                                                     __builtin_fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
        const float amax_b =  // the block's other half sits in lane ^ 1
            __builtin_fmaxf(am, __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(am), 0xB1,
                                                                                  0xF, 0xF, false)));
        float sq = 0.0f;  // Eq. 3
        if (fq.t > 0.0f) {
            const float q0 = amax_b * fq.rt;
            sq = __builtin_fmaf(__builtin_fmaf(-q0, fq.t, amax_b), fq.rt, q0);
            if (!(fq.tfast & (amax_b <= fq.tlim) & ((amax_b == 0.0f) | (amax_b >= 0x1p-100f))))
                sq = div_rn(amax_b, fq.t);
        }
        const uint32_t code = e4m3_encode(sq);
        const float4 e = fq.dtab[code];
        const uint32_t packed = amax_b <= e.z ? quant8_fast(w, e.x, e.y) : quant8(w, e.x);
        *reinterpret_cast<half8_t *>(lds + lds_off(id >> 3, id & 7)) = expand8(packed, e4m3_to_f16x2_over256(code));
    }
}

// ---------------------------------------------------------------- kernel
enum Kind { KIND_NVFP4 = 0, KIND_FUSED = 1, KIND_BF16 = 2 };
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// Register stage of one pipeline step, per operand kind: A then W.
template <class SA, class SW>
struct StagePair {
    SA a;
    SW w;
};
template <int kKind, int EA, int EW>
struct StageSel {
    typedef StagePair<Fp4Stage<EA>, Fp4Stage<EW>> type;
};
template <int EA, int EW>
struct StageSel<KIND_FUSED, EA, EW> {
    typedef StagePair<Bf16Stage<EA>, Fp4Stage<EW>> type;
};
template <int EA, int EW>
struct StageSel<KIND_BF16, EA, EW> {
    typedef StagePair<Bf16Stage<EA>, Bf16Stage<EW>> type;
};

template <int kKind>
struct KindTraits {
    typedef half_t lds_t;
};
template <>
struct KindTraits<KIND_BF16> {
    typedef uint16_t lds_t;
};

// One output tile.  kMode 0 is the interior fast path (whole tile in range,
// K % 64 == 0): no bounds checks, so each pipeline step is one basic block
// the scheduler can interleave (mode 3: the same with global loads).  kMode 1
// (a tile over the M or N edge) keeps that shape, its loads reading zeros
// past the edge; the epilogue checks rows and columns.  kMode 2 checks every
// access (K tails, or a tile whose rows span 2^31 bytes or more).  kMode 4 is
// mode 0 for NVFP4 operands with K % 256 == 0, the block scales fetched per
// group of four K steps.  Operands are prefetched two K steps ahead in
// registers.
template <class C, int kKind, int kOut, int kMode>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, int64_t m0, int64_t n0,
                                          typename KindTraits<kKind>::lds_t *lds) {
    typedef typename KindTraits<kKind>::lds_t lds_t;
    constexpr bool kGuard = kMode == 1 || kMode == 2;  // the epilogue checks rows and columns
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT, TM = C::TM, TN = C::TN;
    constexpr int KS = BK / 16;  // k16 MFMA steps per pipeline step
    auto As = [&](int s) __attribute__((always_inline)) { return lds + s * (BM + BN) * BK; };
    auto Ws = [&](int s) __attribute__((always_inline)) { return lds + s * (BM + BN) * BK + BM * BK; };

    const int KT = (int)((g.K + BK - 1) / BK);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WGN, wn = wave % C::WGN;

    FusedQuant fq{1.0f, 0.0f, 0.0f, 0.0f, false, nullptr};
    if constexpr (kKind == KIND_FUSED) {
        __shared__ float4 dtab[128];
        fq.alpha = *g.a_alpha;
        fq.t = fq.alpha * kQmax;
        fq.rt = fq.t > 0.0f ? div_rn(1.0f, fq.t) : 0.0f;
        fq.tfast = fq.t >= 0x1p-100f && fq.t <= 0x1p100f;
        fq.tlim = fq.t * 0x1p120f;
        fq.dtab = dtab;
        if (threadIdx.x < 128) {
            const float d = fq.alpha * e4m3_decode(threadIdx.x);
            const bool in = d >= 0x1p-90f && d <= 0x1p100f;
            dtab[threadIdx.x] = make_float4(d, in ? div_rn(1.0f, d) : 0.0f, in ? d * 0x1p120f : -1.0f, 0.0f);
        }
        __syncthreads();  // the table is read while the first stage is staged
    }

    typedef typename StageSel<kKind, Part<BM, NT>::EPT, Part<BN, NT>::EPT>::type Stage;

    // Mode 4 (NVFP4, two threads per row and step, K % 256 == 0): the block
    // scales are fetched per group of four steps, 16 bytes per row (the
    // row's two threads load 8 bytes each, one request) instead of 4 bytes
    // per row and step; fetched per step they made half of the loop's L2
    // requests.  A group is loaded two steps before its first fill and
    // unpacked (each thread's 2 bytes of each step, half of them from the
    // partner lane) when its first fill is issued.
    constexpr bool kSB = kMode == 4;
    static_assert(!kSB || (kKind == KIND_NVFP4 && Part<BM, NT>::EPT == 32 && Part<BN, NT>::EPT == 32 && BM == BN),
                  "grouped scales: NVFP4, two threads per row");
    // (resources over the tile's scale rows; built for every mode, used by 4)
    const rsrc_t sra = make_rsrc(g.a_scales + m0 * (g.K >> 4), (uint32_t)(BM * (g.K >> 4)));
    const rsrc_t srw = make_rsrc(g.w_scales + n0 * (g.K >> 4), (uint32_t)(BN * (g.K >> 4)));
    const uint32_t sgo = (uint32_t)Part<BM, NT>::row() * (uint32_t)(g.K >> 4) + 8u * (uint32_t)Part<BM, NT>::part();
    u32x2_t graw_a{0, 0}, graw_w{0, 0}, gpk_a{0, 0}, gpk_w{0, 0};
    auto load_group = [&](int grp) __attribute__((always_inline)) {
        graw_a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(sra, sgo, grp * 16, 0));
        graw_w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(srw, sgo, grp * 16, 0));
    };
    // part 0 holds bytes 0-7 of the group (steps 0, 1), part 1 bytes 8-15;
    // a part's 2 bytes of a step sit at 2 * part within the step's word
    auto unpack = [&](u32x2_t v) __attribute__((always_inline)) {
        const uint32_t ox = (uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        const uint32_t oy = (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0xB1, 0xF, 0xF, false);
        return (threadIdx.x & 1) ? u32x2_t{(ox >> 16) | (oy & 0xFFFF0000u), (v.x >> 16) | (v.y & 0xFFFF0000u)}
                                 : u32x2_t{(v.x & 0xFFFFu) | (v.y << 16), (ox & 0xFFFFu) | (oy << 16)};
    };
    auto group_sc = [&](u32x2_t pk, int kt) __attribute__((always_inline)) {
        return (((kt & 2) ? pk.y : pk.x) >> (16 * (kt & 1))) & 0xFFFFu;
    };

    // load half p (0: A, 1: W) of pipeline step kt into the register stage
    auto load_part = [&](Stage &st, int kt, int p) __attribute__((always_inline)) {
        if (p == 0) {
            if constexpr (kKind == KIND_NVFP4) {
                fp4_load<BM, NT, kMode>(st.a, (const uint8_t *)g.a, g.a_scales, g.M, g.K, m0, kt);
                if constexpr (kSB) st.a.sc = group_sc(gpk_a, kt);
            } else {
                bf16_load<BM, NT, kMode>(st.a, (const uint16_t *)g.a, g.lda, g.M, g.K, m0, kt);
            }
        } else {
            if constexpr (kKind == KIND_BF16) {
                bf16_load<BN, NT, kMode>(st.w, (const uint16_t *)g.w, g.K, g.N, g.K, n0, kt);
            } else {
                fp4_load<BN, NT, kMode>(st.w, (const uint8_t *)g.w, g.w_scales, g.N, g.K, n0, kt);
                if constexpr (kSB) st.w.sc = group_sc(gpk_w, kt);
            }
        }
    };
    // stage quarter q of a register stage into LDS buffer s: A's first and
    // second half of blocks (q = 0, 1), then W's (q = 2, 3)
    auto store_q = [&](const Stage &st, int s, auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        constexpr int h = q & 1;
        if constexpr (q < 2) {
            if constexpr (kKind == KIND_NVFP4) fp4_store<BM, NT, h>(st.a, (half_t *)As(s));
            if constexpr (kKind == KIND_FUSED) fused_store<BM, NT, h>(st.a, (half_t *)As(s), fq);
            if constexpr (kKind == KIND_BF16) bf16_store<BM, NT, h>(st.a, (uint16_t *)As(s));
        } else {
            if constexpr (kKind == KIND_BF16)
                bf16_store<BN, NT, h>(st.w, (uint16_t *)Ws(s));
            else
                fp4_store<BN, NT, h>(st.w, (half_t *)Ws(s));
        }
    };
    auto store_all = [&](const Stage &st, int s) __attribute__((always_inline)) {
        store_q(st, s, std::integral_constant<int, 0>());
        store_q(st, s, std::integral_constant<int, 1>());
        store_q(st, s, std::integral_constant<int, 2>());
        store_q(st, s, std::integral_constant<int, 3>());
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    uint4 af[2][TM], bf[2][TN];
    auto read_frags = [&](int s, int ks, uint4 *fa, uint4 *fb) __attribute__((always_inline)) {
        const lds_t *A = As(s);
        const lds_t *W = Ws(s);
        const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[i] = *reinterpret_cast<const uint4 *>(A + lds_off(wm * C::WM + i * 32 + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[j] = *reinterpret_cast<const uint4 *>(W + lds_off(wn * C::WN + j * 32 + (lane & 31), chunk));
    };
    auto mfmas = [&](const uint4 *fa, const uint4 *fb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (kKind == KIND_BF16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                                        __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j],
                                                                        0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, fa[i]),
                                                                       __builtin_bit_cast(half8_t, fb[j]), acc[i][j],
                                                                       0, 0, 0);
            }
    };
    // Pipeline step kt computes on LDS buffer kt & 1.  Register stage `use`
    // holds step kt + 1 (loaded during the previous step) and is staged into
    // buffer (kt + 1) & 1 over the first three k16 MFMA groups (A's blocks,
    // then W's).  Step kt + 2 is loaded into `fill` before any MFMA, so the
    // loads have the whole step to land, and moved into `use` at the end.
    Stage use, fill;
    // LDS hand-off: this wave's LDS reads and writes complete, then a plain
    // barrier (register prefetches stay in flight across it)
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
        __builtin_amdgcn_s_barrier();
    };
    // The stores into the idle buffer finish by the third k16 group; the
    // barrier then sits before the last group, whose fragments are already in
    // registers, and the next step's first fragments are read under its MFMAs.
    auto step = [&](int kt, bool do_store, bool do_load, bool has_next) __attribute__((always_inline)) {
        const int cur = kt & 1;
        if constexpr (kSB) {
            if (do_load && (kt & 3) == 0) load_group(min((kt >> 2) + 1, (KT >> 2) - 1));
            if (do_load && (kt & 3) == 2) {
                gpk_a = unpack(graw_a);
                gpk_w = unpack(graw_w);
            }
        }
        if (do_load) {
            load_part(fill, kt + 2, 0);
            load_part(fill, kt + 2, 1);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) read_frags(cur, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
            // NVFP4 and fused: keep the next group's fragment reads ahead of
            // this group's MFMAs (the scheduler otherwise sinks each read next
            // to its use and the LDS latency is exposed).  Measured slower for
            // the BF16 kind, which keeps the default schedule.
            if constexpr (kKind != KIND_BF16) __builtin_amdgcn_sched_barrier(0);
            if (do_store) {
                if (ks == 0) store_q(use, cur ^ 1, std::integral_constant<int, 0>());
                if (ks == 1) store_q(use, cur ^ 1, std::integral_constant<int, 1>());
                if (ks == 2) {
                    store_q(use, cur ^ 1, std::integral_constant<int, 2>());
                    store_q(use, cur ^ 1, std::integral_constant<int, 3>());
                }
            }
            if (ks == KS - 1 && has_next) {
                lds_barrier();
                read_frags(cur ^ 1, 0, af[0], bf[0]);
            }
            mfmas(af[ks & 1], bf[ks & 1]);
            // NVFP4: interleave the group's 8 MFMAs with its staging work
            // (three or five VALU operations and one LDS write after each
            // MFMA), so one wave keeps the matrix pipe fed while it expands
            // operands: +1.5-2% over the compiler's grouping (same-process A/B
            // on the Qwen3-8B layers at 8192 tokens; two and four VALU
            // operations per MFMA measured slower, four and six the same)
            // BF16: the same for its staging copies (two or three MFMAs per
            // LDS write): +5% on the Qwen3-8B layers at 8192 tokens
            if constexpr (kKind == KIND_BF16) {
                if (do_store && ks < 3) {
                    if (ks == 2) {
                        static_for<4>([&](auto) __attribute__((always_inline)) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                        });
                    } else {
                        static_for<2>([&](auto) __attribute__((always_inline)) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                        });
                    }
                }
            }
            if constexpr (kKind == KIND_NVFP4) {
                if (do_store && ks < 3) {
                    if (ks == 2) {  // both halves of W
                        static_for<8>([&](auto) __attribute__((always_inline)) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
                        });
                    } else {
                        static_for<8>([&](auto) __attribute__((always_inline)) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                        });
                    }
                }
            }
        }
        if (do_load) use = fill;
    };
    static_assert(KS == 4, "stores are spread over the first three k16 groups");

    if constexpr (kSB) {
        load_group(0);
        gpk_a = unpack(graw_a);
        gpk_w = unpack(graw_w);
    }
    if (KT > 0) {
        load_part(use, 0, 0);
        load_part(use, 0, 1);
        store_all(use, 0);
        if (KT > 1) {
            load_part(use, 1, 0);
            load_part(use, 1, 1);
        }
    }
    __syncthreads();
    if (KT > 0) read_frags(0, 0, af[0], bf[0]);
    int kt = 0;
    for (; kt + 2 < KT; ++kt) step(kt, true, true, true);
    if (kt + 1 < KT) {
        step(kt, true, false, true);
        ++kt;
    }
    if (kt < KT) step(kt, false, false, false);

    // epilogue: y = (acc * alphaA) * alphaW, stored FP32 or BF16 (nearest-even)
    float sa = 1.0f, sw = 1.0f;
    if (kKind != KIND_BF16) {
        sa = *g.a_alpha;
        sw = *g.w_alpha;
    }
    if constexpr (kOut == OUT_NVFP4) {
        // Quantized output for the next layer (Eq. 3 / Eq. 2 with the static
        // output scale).  Each wave stages its results through LDS one 32-row
        // slab at a time, so that a lane then owns whole 16-element blocks of
        // a row: block amax, block scale and the 16 codes are formed in-lane
        // and stored as 8 bytes + 1 scale byte.  N % 16 == 0.
        static_assert(C::WN % 64 == 0 && C::WM % 32 == 0, "quantizing epilogue: wave tiles of 64k columns");
        constexpr int SLD = C::WN + 8;  // padded row stride (floats): the two half-waves hit different banks
        constexpr int BPR = C::WN / 16, NBL = 32 * BPR / 64;  // blocks per slab row, blocks per lane
        const float ya = *g.out_alpha;
        const int64_t ldc = g.N >> 1, lds_ = g.N >> 4;
        uint8_t *codes = reinterpret_cast<uint8_t *>(g.out);
        const float t6 = ya * kQmax, rt6 = t6 > 0.0f ? div_rn(1.0f, t6) : 0.0f;
        const bool tfast = (t6 >= 0x1p-100f) & (t6 <= 0x1p100f);
        float *slab = reinterpret_cast<float *>(lds) + wave * (32 * SLD);
        __syncthreads();  // every wave is done with the operand buffers
        static_for<TM>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            // fragment layout -> row-major slab (32 rows x 128 columns)
            static_for<TN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                static_for<16>([&](auto rc) __attribute__((always_inline)) {
                    constexpr int r = decltype(rc)::value;
                    const int rl = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    slab[rl * SLD + j * 32 + (lane & 31)] = (acc[i][j][r] * sa) * sw;
                });
            });
            // 32 rows x BPR blocks: lane handles blocks lane + 64 q
#pragma unroll
            for (int q = 0; q < NBL; ++q) {
                const int bi = lane + 64 * q, rl = bi / BPR, blk = bi % BPR;
                float v[16];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float4 t = *reinterpret_cast<const float4 *>(slab + rl * SLD + blk * 16 + 4 * e);
                    v[4 * e] = t.x;
                    v[4 * e + 1] = t.y;
                    v[4 * e + 2] = t.z;
                    v[4 * e + 3] = t.w;
                }
                uint32_t am = 0;
                bool tiny = false;  // a nonzero |v| below 2^-100 (outside the fast division's range)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t ab = __float_as_uint(v[e]) & 0x7FFFFFFFu;
                    am = max(am, ab);
                    tiny = tiny | ((ab != 0u) & (ab < 0x0D800000u));  // 2^-100 = 0x0D800000
                }
                const float amax = __uint_as_float(am);
                // Eq. 3 with the tensor-wide reciprocal (Markstein) when it qualifies
                float sq;
                if (__all(tfast & (amax <= t6 * 0x1p120f) & ((amax == 0.0f) | (amax >= 0x1p-100f)))) {
                    const float q0 = amax * rt6;
                    sq = __builtin_fmaf(__builtin_fmaf(-q0, t6, amax), rt6, q0);
                } else {
                    sq = t6 > 0.0f ? div_rn(amax, t6) : 0.0f;
                }
                const uint32_t code = e4m3_encode(sq);
                const float d = ya * e4m3_decode(code);
                // Eq. 2: one reciprocal per block, Markstein per element
                const float rd = d > 0.0f ? div_rn(1.0f, d) : 0.0f;
                float qv[16];
                if (__all((d >= 0x1p-100f) & (d <= 0x1p100f) & !tiny & (amax <= d * 0x1p120f))) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float q0 = v[e] * rd;
                        qv[e] = __builtin_fmaf(__builtin_fmaf(-q0, d, v[e]), rd, q0);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        qv[e] = d > 0.0f ? div_rn(v[e], d) : __uint_as_float(__float_as_uint(v[e]) & 0x80000000u);
                }
                // nearest-even E2M1 with saturation, sign kept (hardware convert)
                uint32_t w0 = 0, w1 = 0;
                w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[0], qv[1], 1.0f, 0);
                w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[2], qv[3], 1.0f, 1);
                w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[4], qv[5], 1.0f, 2);
                w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[6], qv[7], 1.0f, 3);
                w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[8], qv[9], 1.0f, 0);
                w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[10], qv[11], 1.0f, 1);
                w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[12], qv[13], 1.0f, 2);
                w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[14], qv[15], 1.0f, 3);
                const int64_t row = m0 + wm * C::WM + i * 32 + rl, col = n0 + wn * C::WN + blk * 16;
                if ((!kGuard | (row < g.M)) & (!kGuard | (col < g.N))) {
                    uint32_t *cp = reinterpret_cast<uint32_t *>(codes + row * ldc + (col >> 1));
                    cp[0] = w0;
                    cp[1] = w1;
                    g.out_scales[row * lds_ + (col >> 4)] = (uint8_t)code;
                }
            }
        });
        return;
    } else {
        // staged through a per-wave LDS slab (the operand buffers are free
        // once every wave has left the main loop) for 16-byte row stores
        static_assert(NT / 64 * epilogue_slab_floats<TN>() * 4 <= 2 * (BM + BN) * BK * 2, "slabs fit the LDS");
        __syncthreads();
        float *slab = reinterpret_cast<float *>(lds) + wave * epilogue_slab_floats<TN>();
        store_acc_tiles<TM, TN, kOut == OUT_BF16>(acc, sa, sw, slab, g.out, g.ld_out, m0 + wm * C::WM,
                                                  n0 + wn * C::WN, g.M, g.N, g.vec);
        if constexpr (kOut == OUT_F32_AMAX) {
            // max |y| over the wave tile, each y formed as it was stored
            // (elements past the M or N edge are exact zeros)
            static_assert(NT / 64 <= 8, "eight slots per workgroup");
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        m = max(m, __float_as_uint((acc[i][j][r] * sa) * sw) & 0x7FFFFFFFu);
            for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
            if (lane == 0) {
                g.amax_part[(int64_t)blockIdx.x * 8 + wave] = m;
                if (NT / 64 == 4) g.amax_part[(int64_t)blockIdx.x * 8 + 4 + wave] = 0u;
            }
        }
    }
}

template <class C, int kKind, int kOut>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_kernel(GemmArgs g) {
    typedef typename KindTraits<kKind>::lds_t lds_t;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    lds_t *lds = reinterpret_cast<lds_t *>(smem);
    int tm, tn;
    tile_coords<C::BM, C::BN>(g.M, g.N, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    if ((g.K & (BK - 1)) == 0 && g.rows_rsrc) {
        if (m0 + C::BM <= g.M && n0 + C::BN <= g.N) {
            if constexpr (kKind == KIND_NVFP4 && Part<C::BM, C::NT>::EPT == 32) {
                if ((g.K & 255) == 0)
                    gemm_tile<C, kKind, kOut, 4>(g, m0, n0, lds);
                else
                    gemm_tile<C, kKind, kOut, 0>(g, m0, n0, lds);
            } else {
                gemm_tile<C, kKind, kOut, kKind == KIND_FUSED ? 3 : 0>(g, m0, n0, lds);
            }
        }
        else
            gemm_tile<C, kKind, kOut, 1>(g, m0, n0, lds);
    } else {
        gemm_tile<C, kKind, kOut, 2>(g, m0, n0, lds);
    }
}

template <class C, int kKind, int kOut>
hipError_t launch_cfg(const GemmArgs &g, hipStream_t s) {
    const int64_t nb = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN);
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const size_t lds_bytes = (size_t)2 * (C::BM + C::BN) * BK * 2;
    auto kern = gemm_kernel<C, kKind, kOut>;
    GemmArgs ga = g;
    const int64_t a_row = kKind == KIND_NVFP4 ? g.K / 2 : g.lda * 2, w_row = kKind == KIND_BF16 ? g.K * 2 : g.K / 2;
    ga.rows_rsrc = C::BM * a_row < (int64_t(1) << 31) && C::BN * w_row < (int64_t(1) << 31);
    ga.vec = kOut != OUT_NVFP4 && epilogue_vec_ok(g.out, g.ld_out, kOut == OUT_BF16 ? 2 : 4);
    static std::atomic<uint32_t> attr_done{0};
    if (hipError_t e = set_dyn_lds_once(attr_done, (const void *)kern, (int)lds_bytes); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(C::NT), lds_bytes, s, ga);
    return hipGetLastError();
}

// Tile choice: NVFP4_GEMM_TILE=big4|big8|small overrides (tuning knob);
// default: a 256 x 256 tile once its tiles occupy at least 192 of the 256
// CUs (one round), else 128 x 128.  Measured per layer at 512-4096 tokens:
// gate_up at 512 tokens (192 large tiles) 125 -> 102 us and qkv at 2048
// (192) 117 -> 97 us on the large tile, while at 128 large tiles (o and down
// at 2048) the small tile stays 10-15% faster; the BF16 kind alike.
// The variable is read once per process (a function-local static: its
// initialisation is thread-safe).
int tile_override() {
    static const int v = [] {
        const char *e = getenv("NVFP4_GEMM_TILE");
        return !e ? 0 : !strcmp(e, "big4") ? 1 : !strcmp(e, "big8") ? 2 : !strcmp(e, "small") ? 3 : 0;
    }();
    return v;
}

template <class C, int kKind>
hipError_t launch_out(const GemmArgs &g, int out_type, hipStream_t s) {
    if constexpr (kKind == KIND_NVFP4) {
        if (out_type == OUT_NVFP4) return launch_cfg<C, kKind, OUT_NVFP4>(g, s);
        if (out_type == OUT_F32_AMAX) return launch_cfg<C, kKind, OUT_F32_AMAX>(g, s);
    }
    if (out_type == OUT_NVFP4 || out_type == OUT_F32_AMAX) return hipErrorInvalidValue;
    return out_type == OUT_BF16 ? launch_cfg<C, kKind, OUT_BF16>(g, s) : launch_cfg<C, kKind, OUT_F32>(g, s);
}

// Tile choice: 1 = 4-wave 256 x 256, 2 = 8-wave 256 x 256, 3 = 128 x 128.
int tile_choice(int64_t M, int64_t N) {
    const int t = tile_override();
    return t ? t : ((M + 255) / 256) * ((N + 255) / 256) >= 192 ? 2 : 3;
}

template <int kKind>
hipError_t launch(const GemmArgs &g, int out_type, hipStream_t s) {
    int t = tile_choice(g.M, g.N);
    // the fused prologue needs more registers than 8 waves leave the main
    // loop (it spills there): the 4-wave 256 x 256 tile (512 registers per
    // lane) runs it (an explicit NVFP4_GEMM_TILE=big8 still takes 8 waves)
    if (t == 2 && kKind == KIND_FUSED && tile_override() == 0) t = 1;
    if (t == 1) return launch_out<BigTile, kKind>(g, out_type, s);
    if (t == 2) return launch_out<BigTile8, kKind>(g, out_type, s);
    return launch_out<SmallTile, kKind>(g, out_type, s);
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha, int64_t M,
                             int64_t N, int64_t K, void *out, int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, 0, out, ld_out, nullptr, nullptr};
    return launch<KIND_NVFP4>(g, out_type, s);
}

hipError_t launch_gemm_nvfp4_quant_out(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                       const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                       int64_t M, int64_t N, int64_t K, uint8_t *y_codes, uint8_t *y_scales,
                                       const float *y_alpha, hipStream_t s) {
    GemmArgs g{a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, 0, y_codes, N / 2, y_scales, y_alpha};
    return launch<KIND_NVFP4>(g, OUT_NVFP4, s);
}

hipError_t launch_gemm_nvfp4_f32_amax(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_alpha,
                                      const uint8_t *w_codes, const uint8_t *w_scales, const float *w_alpha,
                                      int64_t M, int64_t N, int64_t K, float *y, uint32_t *parts, hipStream_t s) {
    GemmArgs g{a_codes, a_scales, a_alpha, w_codes, w_scales, w_alpha, M, N, K, 0, y, N, nullptr, nullptr};
    g.amax_part = parts;
    return launch<KIND_NVFP4>(g, OUT_F32_AMAX, s);
}

int64_t gemm_amax_parts(int64_t M, int64_t N) {
    const int64_t b = tile_choice(M, N) == 3 ? 128 : 256;
    return ((M + b - 1) / b) * ((N + b - 1) / b) * 8;
}

int64_t gemm_amax_parts_bound(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128) * 8; }

hipError_t launch_gemm_fused(const uint16_t *x, int64_t ld_x, const float *a_alpha, const uint8_t *w_codes,
                             const uint8_t *w_scales, const float *w_alpha, int64_t M, int64_t N, int64_t K,
                             void *out, int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{x, nullptr, a_alpha, w_codes, w_scales, w_alpha, M, N, K, ld_x, out, ld_out, nullptr, nullptr};
    return launch<KIND_FUSED>(g, out_type, s);
}

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                            int out_type, int64_t ld_out, hipStream_t s) {
    GemmArgs g{a, nullptr, nullptr, w, nullptr, nullptr, M, N, K, K, out, ld_out, nullptr, nullptr};
    return launch<KIND_BF16>(g, out_type, s);
}

}  // namespace nvfp4
