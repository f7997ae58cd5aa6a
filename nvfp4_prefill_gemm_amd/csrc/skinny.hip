// BF16 decode GEMM for small batches (M <= 64): Y[M, N] = X[M, K] * W[N, K]^T.
//
// Decode keeps the original BF16 weights (Mix-Quant Section 3.3,
// "Prefill-Decode Disaggregation Deployment") and is bound by streaming W
// from HBM: 2*N*K bytes against 2*M*N*K flops.  Each workgroup owns a strip
// of NG*16 weight rows; its waves split K in 32-wide steps (interleaved, so
// the waves of a workgroup read neighbouring 64-byte pieces of the same
// rows), keep U steps of loads in flight, and run 16x16x32 BF16 MFMAs with
// X zero-padded to MG*16 rows.  The per-wave partial tiles are summed
// through LDS at the end.
#include <stdlib.h>
#include <string.h>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __attribute__((ext_vector_type(4))) float f4_t;

template <int MG, int NG, int WAVES, int U, bool kOutBf16>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                            int64_t M, int64_t N, int64_t K, void *__restrict__ out,
                                                            int64_t ld_out) {
    __shared__ float red[WAVES][MG][NG][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * (NG * 16);
    const int kq = (lane >> 4) * 8;
    const int64_t KS = (K + 31) >> 5;

    f4_t acc[MG][NG];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t *wr[NG];
    bool wv[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int64_t n = n0 + j * 16 + (lane & 15);
        wv[j] = n < N;
        wr[j] = w + (wv[j] ? n : 0) * K;
    }
    const uint16_t *xr[MG];
    bool xv[MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) {
        const int64_t m = i * 16 + (lane & 15);
        xv[i] = m < M;
        xr[i] = x + (xv[i] ? m : 0) * K;
    }

    for (int64_t ks0 = wave; ks0 < KS; ks0 += (int64_t)WAVES * U) {
        uint4 bw[U][NG], ax[U][MG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = (ks0 + (int64_t)u * WAVES) * 32 + kq;
            const bool kin = k + 8 <= K;
#pragma unroll
            for (int j = 0; j < NG; ++j)
                bw[u][j] = (kin && wv[j]) ? load_nt16(wr[j] + k)
                                          : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < MG; ++i)
                ax[u][i] = (kin && xv[i]) ? *reinterpret_cast<const uint4 *>(xr[i] + k) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < MG; ++i)
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[u][i]),
                                                                        __builtin_bit_cast(bf16x8_t, bw[u][j]),
                                                                        acc[i][j], 0, 0, 0);
    }

#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][i][j][lane][r] = acc[i][j][r];
    __syncthreads();

    // out[m = i*16 + (l>>4)*4 + r][n = n0 + j*16 + (l & 15)]
    constexpr int TOTAL = MG * NG * 64 * 4;
    for (int idx = threadIdx.x; idx < TOTAL; idx += WAVES * 64) {
        const int r = idx & 3, l = (idx >> 2) & 63, j = (idx >> 8) % NG, i = (idx >> 8) / NG;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) s += red[v][i][j][l][r];
        const int64_t m = i * 16 + (l >> 4) * 4 + r, n = n0 + j * 16 + (l & 15);
        if (m < M && n < N) {
            if (kOutBf16)
                reinterpret_cast<uint16_t *>(out)[m * ld_out + n] = (uint16_t)f32_to_bf16_bits(s);
            else
                reinterpret_cast<float *>(out)[m * ld_out + n] = s;
        }
    }
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

__global__ void fill_zero_kernel(uint8_t *out, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
        for (int64_t c = threadIdx.x; c < row_bytes; c += blockDim.x) out[r * ld_bytes + c] = 0;
}

}  // namespace

// NVFP4_SKINNY_CFG=<waves>x<unroll> overrides the decode kernel shape (tuning knob).
int skinny_cfg() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("NVFP4_SKINNY_CFG");
        v = !e ? 0 : !strcmp(e, "8x4") ? 1 : !strcmp(e, "16x4") ? 2 : !strcmp(e, "16x8") ? 3 : !strcmp(e, "8x8") ? 4 : 0;
    }
    return v;
}

template <int MG, int NG>
hipError_t launch_mg(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out, int out_type,
                     int64_t ld_out, hipStream_t s) {
    switch (skinny_cfg()) {
        case 1: return launch_cfg<MG, NG, 8, 4>(a, w, M, N, K, out, out_type, ld_out, s);
        case 3: return launch_cfg<MG, NG, 16, 8>(a, w, M, N, K, out, out_type, ld_out, s);
        case 4: return launch_cfg<MG, NG, 8, 8>(a, w, M, N, K, out, out_type, ld_out, s);
        default: return launch_cfg<MG, NG, 16, 4>(a, w, M, N, K, out, out_type, ld_out, s);
    }
}

hipError_t launch_skinny_bf16(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K, void *out,
                              int out_type, int64_t ld_out, hipStream_t s) {
    if (M <= 16) return launch_mg<1, 1>(a, w, M, N, K, out, out_type, ld_out, s);
    if (M <= 32) return launch_mg<2, 1>(a, w, M, N, K, out, out_type, ld_out, s);
    if (M <= 64) return launch_mg<4, 1>(a, w, M, N, K, out, out_type, ld_out, s);
    return hipErrorInvalidValue;
}

hipError_t launch_fill_zero(void *out, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t g = rows < 4096 ? rows : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, s, (uint8_t *)out, rows, cols * elem_bytes,
                       ld * elem_bytes);
    return hipGetLastError();
}

}  // namespace nvfp4
