// Output epilogue shared by the tile GEMMs: a wave's 32x32 MFMA accumulator
// tiles are staged through a per-wave LDS slab so that each lane then writes
// eight consecutive output columns of one row (one 16-byte store for BF16, two
// for FP32) instead of one 2- or 4-byte value per accumulator register.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// LDS floats per wave for a wave tile of TN 32-column MFMA tiles: one 32-row
// slab, rows padded by 8 floats (the two half-waves of a slab write, four
// rows apart, then fall on different banks).
template <int TN>
constexpr int epilogue_slab_floats() {
    return 32 * (TN * 32 + 8);
}

// y = (acc * sa) * sw of the wave tile whose top-left output element is
// (row0, col0), stored to out [M, ld_out] as FP32 or BF16 (nearest-even).
// The 32x32 MFMA result layout puts element r of lane l of tile (i, j) at
// row i*32 + (r/4)*8 + (l/32)*4 + r%4, column j*32 + l%32.  vec: out and
// ld_out allow 16-byte stores; rows past M and columns past N are skipped.
// The caller has finished every other use of `slab` (a workgroup barrier
// after the main loop); each wave only reads back its own writes.
template <int TM, int TN, bool kOutBf16>
__device__ __forceinline__ void store_acc_tiles(const f32x16_t (&acc)[TM][TN], float sa, float sw,
                                                float *__restrict__ slab, void *__restrict__ out, int64_t ld_out,
                                                int64_t row0, int64_t col0, int64_t M, int64_t N, bool vec) {
    constexpr int W = TN * 32, SLD = W + 8;
    constexpr int LPR = W / 8;        // lanes per slab row (8 columns each)
    constexpr int RPP = 64 / LPR;     // slab rows per pass
    static_assert(64 % LPR == 0 && 32 % RPP == 0, "wave tile width");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                slab[rl * SLD + j * 32 + (lane & 31)] = (acc[i][j][r] * sa) * sw;
            }
#pragma unroll
        for (int p = 0; p < 32 / RPP; ++p) {
            const int rl = p * RPP + lane / LPR, c = (lane % LPR) * 8;
            const float4 lo = *reinterpret_cast<const float4 *>(slab + rl * SLD + c);
            const float4 hi = *reinterpret_cast<const float4 *>(slab + rl * SLD + c + 4);
            const int64_t row = row0 + i * 32 + rl, col = col0 + c;
            if (row >= M) continue;
            if (kOutBf16) {
                __bf16 *o = reinterpret_cast<__bf16 *>(out) + row * ld_out + col;
                const bf16x2_t b0 = __builtin_convertvector((f32x2_t{lo.x, lo.y}), bf16x2_t);
                const bf16x2_t b1 = __builtin_convertvector((f32x2_t{lo.z, lo.w}), bf16x2_t);
                const bf16x2_t b2 = __builtin_convertvector((f32x2_t{hi.x, hi.y}), bf16x2_t);
                const bf16x2_t b3 = __builtin_convertvector((f32x2_t{hi.z, hi.w}), bf16x2_t);
                if (vec && col + 8 <= N) {
                    *reinterpret_cast<uint4 *>(o) =
                        make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                                   __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
                } else {
                    const __bf16 v[8] = {b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < N) o[e] = v[e];
                }
            } else {
                float *o = reinterpret_cast<float *>(out) + row * ld_out + col;
                if (vec && col + 8 <= N) {
                    reinterpret_cast<float4 *>(o)[0] = lo;
                    reinterpret_cast<float4 *>(o)[1] = hi;
                } else {
                    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < N) o[e] = v[e];
                }
            }
        }
    }
}

// 16-byte stores need a 16-byte aligned base and row pitch.
inline bool epilogue_vec_ok(const void *out, int64_t ld_out, int elem_bytes) {
    return (reinterpret_cast<uintptr_t>(out) & 15) == 0 && (ld_out * elem_bytes) % 16 == 0;
}

}  // namespace nvfp4
