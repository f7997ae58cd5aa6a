// Device-side NVFP4 format helpers for gfx950.
//
// NVFP4 (Mix-Quant, Section 3.3): E2M1 element codes, one FP8 E4M3 scale per
// 16 elements, one FP32 tensor scale.  The rounding here is done with IEEE
// bit manipulation and gfx950's FP4/FP8 converts; every function is
// round-to-nearest, ties-to-even, on the FP32 value it is given.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// 16-byte streaming load (data read once: non-temporal hint).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr float kQmax = 6.0f;         // largest finite E2M1 magnitude
constexpr float kE4M3Max = 448.0f;    // largest finite E4M3 ("FN") value
constexpr float kAlphaDen = 2688.0f;  // kQmax * kE4M3Max

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// FP32 -> BF16 bits, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eq. 3's projection onto the E4M3 grid: nearest-even, saturating at 448,
// for s >= 0; returns the 8-bit code (sign bit clear).  gfx950's FP32 -> FP8
// convert produces OCP E4M3 ("FN") with nearest-even rounding, subnormals
// (the m * 2^-9 grid below 2^-6) included; the clamp to 448 first handles
// saturation, and maps +inf and NaN (minNum) to 448, code 0x7E.  On the GPU
// this agreed with a bit-manipulation encoder (3 mantissa bits kept, nearest-
// even, a carry moving into the exponent; the subnormal grid by rint) on all
// 2^31 non-negative FP32 bit patterns.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s, kE4M3Max), 0.0f, 0, false);
}

// E4M3 code (sign clear) -> FP32 value, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Correctly rounded FP32 division (IEEE), independent of fast-math flags.
__device__ __forceinline__ float div_rn(float x, float y) { return __fdiv_rn(x, y); }

// RN(a / d) for a >= 0 given r = RN(1/d), by Markstein's correction under the
// conditions stated for quant8 below, else by the IEEE division.
__device__ __forceinline__ float div_rn_recip(float a, float d, float r) {
    if (d >= 0x1p-100f && d <= 0x1p100f && (a == 0.0f || a >= 0x1p-100f) && a <= d * 0x1p120f) {
        const float q0 = a * r;
        return __builtin_fmaf(__builtin_fmaf(-q0, d, a), r, q0);
    }
    return div_rn(a, d);
}

// Eq. 2 for 8 consecutive elements of one block: w[i] holds elements 2i
// (low half) and 2i + 1 (high half) as BF16 bits; d = fl32(alpha * sigma).
// Returns the 8 E2M1 codes packed, element i in nibble i.
//
// |x| / d is formed with Markstein's correction: r = RN(1/d) (one IEEE
// division), q0 = RN(|x| r), then RN(q0 + (|x| - q0 d) r) with both steps as
// fused multiply-adds equals RN(|x| / d) when d, 1/d, x and the quotient stay
// clear of underflow and overflow; d in [2^-100, 2^100], |x| >= 2^-100 (or
// x == 0) and |x| <= d * 2^120 qualify (checked against the IEEE quotient on
// 2.9e8 random BF16 and 2.5e8 random FP32 numerators on a CPU), and anything
// else takes the IEEE division.  The magnitude is rounded to E2M1 by
// the hardware FP32 -> FP4 convert (nearest-even with saturation at 6: it
// agrees on every FP32 bit pattern with the ladder that counts the tie
// points 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 passed, ties to the even
// mantissa) and the sign is copied from x, which is the sign of x / d.
__device__ __forceinline__ uint32_t quant8(const uint32_t w[4], float d) {
    uint32_t signs = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) signs |= (((w[i] >> 15) & 1u) << (8 * i + 3)) | (((w[i] >> 31) & 1u) << (8 * i + 7));
    if (!(d > 0.0f)) return signs;  // zero divisor: signed zeros
    // a BF16 magnitude m is "tiny" when 0 < m < 2^-100 (exponent field < 27)
    bool fast = d >= 0x1p-100f && d <= 0x1p100f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        fast = fast && (lo - 1u >= (27u << 7) - 1u) && (hi - 1u >= (27u << 7) - 1u);
    }
    float a[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[2 * i] = bf16_bits_to_f32(w[i] & 0x7FFFu);
        a[2 * i + 1] = bf16_bits_to_f32((w[i] >> 16) & 0x7FFFu);
    }
    const float lim = d * 0x1p120f;  // quotient bound (inf for d >= 2^8: no bound needed)
#pragma unroll
    for (int i = 0; i < 8; ++i) fast = fast && a[i] <= lim;
    if (fast) {
        const float r = div_rn(1.0f, d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q0 = a[i] * r;
            a[i] = __builtin_fmaf(__builtin_fmaf(-q0, d, a[i]), r, q0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = div_rn(a[i], d);
    }
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[0], a[1], 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[2], a[3], 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[4], a[5], 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, a[6], a[7], 1.0f, 3);
    return packed | signs;
}

// quant8 on its fast path, with r = RN(1/d) supplied: for d in
// [2^-90, 2^100] and every |x| <= d * 2^120, Markstein's correction on the
// signed values, then the hardware convert, gives the codes of the IEEE
// quotient.  The residual is formed negated, e = RN(q0 d - x), and the
// quotient as RN(q0 - e r): for x = -0 that gives -0 (code 0x8) where the
// usual order gives +0.  A CPU run over every finite BF16 numerator against
// 8192 divisors in that range found no code different from the IEEE
// quotient's.  Numerators below 2^-100 need no special case: with d >= 2^-90
// their quotients stay far below 0.25, the first rounding step.
__device__ __forceinline__ uint32_t quant8_fast(const uint32_t w[4], float d, float r) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        q[2 * i] = __uint_as_float(w[i] << 16);
        q[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = q[i], q0 = x * r;
        const float e = __builtin_fmaf(q0, d, -x);
        q[i] = __builtin_fmaf(-e, r, q0);
    }
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, q[0], q[1], 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, q[2], q[3], 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, q[4], q[5], 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, q[6], q[7], 1.0f, 3);
    return packed;
}

// Raw buffer loads: a resource covers [base, base + bytes); loads at offsets
// past the end return zeros without touching memory, so guarded loads need
// no branch.  Word 3 of the resource is the gfx9-family default.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kBufOOB = 0x80000000u;  // an offset past every resource used here
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
typedef __attribute__((ext_vector_type(2))) int i32x2_buf_t;
__device__ __forceinline__ void buf_store8(uint32_t lo, uint32_t hi, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(i32x2_buf_t{(int)lo, (int)hi}, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store1(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, off, 0, 0);
}

// 8 E2M1 codes (one 32-bit word, element 0 in the low nibble) times sigma ->
// 8 FP16 values, exactly.  The hardware converts FP4 pairs to FP16 with a
// power-of-two scale of 2^8; sig2 holds sigma * 2^-8 in both halves, and one
// packed FP16 multiply forms q * sigma.  Every factor is exact in FP16 and so
// is the product (q * sigma has <= 6 significant bits, in [2^-10, 2688]).
__device__ __forceinline__ half8_t expand8(uint32_t w, half2_t sig2) {
    half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * sig2;
    half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * sig2;
    half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * sig2;
    half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * sig2;
    return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// sigma * 2^-8 as FP16, in both halves, from an E4M3 code (sign clear).
// Read as FP16 bits, code << 7 lines E4M3's exponent field up with FP16's
// (bias 15 = 7 + 8) and its three mantissa bits with FP16's top three, and
// E4M3 subnormals m * 2^-9 land on FP16 subnormals m * 2^-17; so the value is
// exactly sigma * 2^-8 for every finite code, with no branch.
__device__ __forceinline__ half2_t e4m3_to_f16x2_over256(uint32_t c) {
    return __builtin_bit_cast(half2_t, (c << 7) | (c << 23));
}

}  // namespace nvfp4
