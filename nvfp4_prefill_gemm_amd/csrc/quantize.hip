// BF16 -> NVFP4 activation quantizer for gfx950 (Mix-Quant Section 3.3,
// Eq. 2 and Eq. 3).  Two passes when the tensor scale is dynamic:
//   1. amax_partials: every workgroup streams its rows with 16-byte loads and
//      writes one partial max |x| (as FP32 bits; non-negative floats order
//      like their bit patterns, so an integer max is exact).
//   2. quantize: every workgroup folds the partials into alpha, then each
//      lane takes 8 consecutive elements (one 16-byte load); lanes 2j and
//      2j+1 share one 16-element block and exchange their half-block maxima
//      with a DPP swap.  Codes leave as one 4-byte store per lane (coalesced),
//      the E4M3 scale as one byte per lane pair.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxParts = 1024;
// Work item of both passes: kSeg 8-element groups (2048 elements) of one row,
// kU 16-byte loads in flight per lane; short rows give one item each, long
// rows several, so small batches still spread over many waves.
constexpr int kU = 4;
constexpr int64_t kSeg = 64 * kU;

typedef __attribute__((ext_vector_type(2))) unsigned short ushort2_t;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

// max over the two BF16 magnitudes packed in w, per 16-bit half
__device__ __forceinline__ ushort2_t abs_bf16x2(uint32_t w) {
    w &= 0x7FFF7FFFu;
    return __builtin_bit_cast(ushort2_t, w);
}

__global__ __launch_bounds__(kThreads) void amax_partials_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                 int64_t cols, int64_t ld,
                                                                 uint32_t *__restrict__ partials) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    ushort2_t m = {0, 0};
    const int64_t octs = cols >> 3;
    const int64_t nseg = (octs + kSeg - 1) / kSeg;
    const int64_t items = rows * nseg;
    for (int64_t it = (int64_t)blockIdx.x * kWaves + wave; it < items; it += (int64_t)gridDim.x * kWaves) {
        const int64_t r = it / nseg, o0 = (it - r * nseg) * kSeg + lane;
        const uint4 *xr = reinterpret_cast<const uint4 *>(x + r * ld);
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = (o0 + 64 * u < octs) ? load_nt16(xr + o0 + 64 * u) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].x));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].y));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].z));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].w));
        }
    }
    uint32_t mm = max((uint32_t)m.x, (uint32_t)m.y) << 16;  // FP32 bits of the BF16 max
    mm = wave_max_u32(mm);
    __shared__ uint32_t red[kWaves];
    if (lane == 0) red[wave] = mm;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = red[0];
        for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
        partials[blockIdx.x] = t;
    }
}

__device__ __forceinline__ float alpha_from_partials(const uint32_t *__restrict__ partials, int nparts) {
    __shared__ uint32_t red[kWaves];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) m = max(m, partials[i]);
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t t = red[0];
    for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
    return div_rn(__uint_as_float(t), kAlphaDen);
}

__global__ __launch_bounds__(kThreads) void alpha_kernel(const uint32_t *__restrict__ partials, int nparts,
                                                         float *__restrict__ alpha) {
    float a = alpha_from_partials(partials, nparts);
    if (threadIdx.x == 0) *alpha = a;
}

template <bool kDynamic>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld, uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales, float *__restrict__ alpha_io,
                                                            const uint32_t *__restrict__ partials, int nparts) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t octs = cols >> 3;  // 8-element groups per row; even, so pairs never straddle rows
    const int64_t nseg = (octs + kSeg - 1) / kSeg;
    const int64_t items = rows * nseg, stride = (int64_t)gridDim.x * kWaves;
    auto load_item = [&](int64_t it, uint4 *v) __attribute__((always_inline)) {
        const int64_t r = it / nseg, o0 = (it - r * nseg) * kSeg + lane;
        const uint4 *xr = reinterpret_cast<const uint4 *>(x + r * ld);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = (it < items && o0 + 64 * u < octs) ? load_nt16(xr + o0 + 64 * u) : make_uint4(0, 0, 0, 0);
    };
    // the first item's loads are issued before the tensor scale is reduced
    int64_t it = (int64_t)blockIdx.x * kWaves + wave;
    uint4 v[kU];
    load_item(it, v);
    float alpha;
    if (kDynamic) {
        alpha = alpha_from_partials(partials, nparts);
        if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_io = alpha;
    } else {
        alpha = *alpha_io;
    }
    for (; it < items; it += stride) {
        if (it != (int64_t)blockIdx.x * kWaves + wave) load_item(it, v);
        const int64_t r = it / nseg, o0 = (it - r * nseg) * kSeg + lane;
        uint32_t *cr = reinterpret_cast<uint32_t *>(codes + r * (cols >> 1));
        uint8_t *sr = scales + r * (cols >> 4);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t o = o0 + 64 * u;
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t am = 0;  // bit pattern of max |x| over this lane's 8 elements
#pragma unroll
            for (int i = 0; i < 4; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
            // partner lane (o ^ 1) holds the other half of the 16-element block
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xB1, 0xF, 0xF, false);
            const BlockScale bs = block_scale(bf16_bits_to_f32(max(am, other)), alpha);
            if (o < octs) {
                cr[o] = quant8(w, bs.d);
                if ((o & 1) == 0) sr[o >> 1] = (uint8_t)bs.code;
            }
        }
    }
}

int64_t quant_items(int64_t rows, int64_t cols) { return rows * (((cols >> 3) + kSeg - 1) / kSeg); }

int quant_grid(int64_t rows, int64_t cols) {
    int64_t g = (quant_items(rows, cols) + kWaves - 1) / kWaves;
    if (g > 65536) g = 65536;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace

int amax_parts(int64_t rows, int64_t cols) {
    int64_t g = (quant_items(rows, cols) + kWaves - 1) / kWaves;
    if (g > kMaxParts) g = kMaxParts;
    return (int)(g < 1 ? 1 : g);
}

hipError_t launch_amax_partials(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint32_t *partials,
                                int nparts, hipStream_t s) {
    hipLaunchKernelGGL(amax_partials_kernel, dim3(nparts), dim3(kThreads), 0, s, x, rows, cols, ld, partials);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint8_t *scales, float *alpha, int dynamic, const uint32_t *partials, int nparts,
                           hipStream_t s) {
    dim3 grid(quant_grid(rows, cols)), block(kThreads);
    if (dynamic)
        hipLaunchKernelGGL(quantize_kernel<true>, grid, block, 0, s, x, rows, cols, ld, codes, scales, alpha,
                           partials, nparts);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, grid, block, 0, s, x, rows, cols, ld, codes, scales, alpha,
                           partials, nparts);
    return hipGetLastError();
}

hipError_t launch_alpha_from_partials(const uint32_t *partials, int nparts, float *alpha, hipStream_t s) {
    hipLaunchKernelGGL(alpha_kernel, dim3(1), dim3(kThreads), 0, s, partials, nparts, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
