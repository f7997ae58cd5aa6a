// BF16 -> NVFP4 activation quantizer for gfx950 (Mix-Quant Section 3.3,
// Eq. 2 and Eq. 3).  Two passes when the tensor scale is dynamic:
//   1. amax_partials: every workgroup streams its rows with 16-byte loads and
//      writes one partial max |x| (as FP32 bits; non-negative floats order
//      like their bit patterns, so an integer max is exact).
//   2. quantize: every workgroup folds the partials into alpha, then each
//      lane takes whole 16-element blocks (two 16-byte loads each), so a
//      block's amax and scale are formed once, in one lane.  Codes leave as
//      one 8-byte store per block, the E4M3 scale as one byte.  The grid
//      holds only as many workgroups as are resident at once; each wave
//      walks its items with the next item's loads in flight.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxParts = 1024;
// Work item of both passes: kSeg 8-element groups (2048 elements) of one row,
// kU 16-byte loads per lane; short rows give one item each, long rows
// several, so small batches still spread over many waves.
constexpr int kU = 4;
constexpr int64_t kSeg = 64 * kU;
constexpr int kBlk = 2;  // quantize pass: 16-element blocks per lane and item (2048 elements)
static_assert(kSeg * 8 == 64 * 16 * kBlk, "both passes share the item size");

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

// LDS hand-off that waits only for this wave's LDS operations, so global
// loads already issued stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// This thread's share of the max over the amax partials (FP32 bits).
__device__ __forceinline__ uint32_t partials_max(const uint32_t *__restrict__ partials, int nparts) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) m = max(m, partials[i]);
    return m;
}

// alpha = amax / 2688 from every thread's partial max (workgroup-wide).
__device__ __forceinline__ float alpha_from_max(uint32_t m) {
    __shared__ uint32_t red[kWaves];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    lds_barrier();
    uint32_t t = red[0];
    for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
    return div_rn(__uint_as_float(t), kAlphaDen);
}

__device__ __forceinline__ float alpha_from_partials(const uint32_t *__restrict__ partials, int nparts) {
    return alpha_from_max(partials_max(partials, nparts));
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
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // 32-bit item arithmetic: the host guarantees items < 2^31 and cols < 2^30
    const uint32_t octs = (uint32_t)(cols >> 3);  // 8-element groups per row; even, so pairs never straddle rows
    const uint32_t nseg = (octs + kSeg - 1) / kSeg;
    const uint32_t items = (uint32_t)rows * nseg, nw = gridDim.x * kWaves;
    // Every item is one wave's (row, segment): buffer resources over that row
    // of X, codes and scales (empty past the last item) turn out-of-range
    // loads into zeros and drop out-of-range stores, without branches.
    // Lane l of an item owns whole 16-element blocks: elements
    // seg * 2048 + j * 1024 + 16 l .. + 16 for j = 0, 1 (two 16-byte loads each).
    auto load_item = [&](uint32_t it, uint4 *v) __attribute__((always_inline)) {
        const bool ok = it < items;
        const uint32_t r = ok ? it / nseg : 0u, e0 = (it - r * nseg) * (kSeg * 8) + lane * 16u;
        const rsrc_t xs = make_rsrc(x + (int64_t)r * ld, ok ? (uint32_t)cols * 2u : 0u);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            v[2 * j] = buf_load16(xs, (e0 + 1024u * j) * 2u);
            v[2 * j + 1] = buf_load16(xs, (e0 + 1024u * j) * 2u + 16u);
        }
    };
    uint32_t it = blockIdx.x * kWaves + wave;
    // the tensor scale's inputs are read first, then the first item's loads
    // are issued, so waiting for the former leaves the latter in flight
    // (nparts <= kMaxParts: at most kMaxParts / kThreads partials per thread,
    // loaded without branches; entries past nparts read as zero)
    constexpr int kPartsPerThread = kMaxParts / kThreads;
    uint32_t pv[kPartsPerThread];
    if (kDynamic) {
        const rsrc_t ps = make_rsrc(partials, (uint32_t)nparts * 4u);
#pragma unroll
        for (int j = 0; j < kPartsPerThread; ++j)
            pv[j] = __builtin_amdgcn_raw_buffer_load_b32(ps, (threadIdx.x + j * kThreads) * 4u, 0, 0);
    }
    const float alpha_in = kDynamic ? 0.0f : *alpha_io;
    asm volatile("" ::: "memory");
    uint4 va[2 * kBlk], vb[2 * kBlk];
    load_item(it, va);
    float alpha = alpha_in;
    if (kDynamic) {
        uint32_t pmax = 0;
#pragma unroll
        for (int j = 0; j < kPartsPerThread; ++j) pmax = max(pmax, pv[j]);
        alpha = alpha_from_max(pmax);
        if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_io = alpha;
    }
    const float t = alpha * kQmax;
    const float rt = t > 0.0f ? div_rn(1.0f, t) : 0.0f;
    // Per E4M3 scale code: the divisor d = fl32(alpha * sigma), RN(1/d), and
    // the largest |x| the fast path of quant8_fast takes (-1 when d is
    // outside [2^-90, 2^100], zero included, so those blocks take quant8).
    __shared__ float4 dtab[128];
    if (threadIdx.x < 128) {
        const float d = alpha * e4m3_decode(threadIdx.x);
        const bool in = d >= 0x1p-90f && d <= 0x1p100f;
        dtab[threadIdx.x] = make_float4(d, in ? div_rn(1.0f, d) : 0.0f, in ? d * 0x1p120f : -1.0f, 0.0f);
    }
    lds_barrier();
    auto quant_item = [&](uint32_t it, const uint4 *v) __attribute__((always_inline)) {
        const bool ok = it < items;
        const uint32_t r = ok ? it / nseg : 0u, e0 = (it - r * nseg) * (kSeg * 8) + lane * 16u;
        const rsrc_t cs = make_rsrc(codes + (int64_t)r * (cols >> 1), ok ? (uint32_t)(cols >> 1) : 0u);
        const rsrc_t ss = make_rsrc(scales + (int64_t)r * (cols >> 4), ok ? (uint32_t)(cols >> 4) : 0u);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const uint32_t el = e0 + 1024u * j;
            const uint32_t w[8] = {v[2 * j].x,     v[2 * j].y,     v[2 * j].z,     v[2 * j].w,
                                   v[2 * j + 1].x, v[2 * j + 1].y, v[2 * j + 1].z, v[2 * j + 1].w};
            uint32_t am = 0;  // bit pattern of max |x| over the block
#pragma unroll
            for (int i = 0; i < 8; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
            const float amax_b = bf16_bits_to_f32(am);
            const uint32_t code = e4m3_encode(t > 0.0f ? div_rn_recip(amax_b, t, rt) : 0.0f);  // Eq. 3
            const float4 e = dtab[code];
            uint32_t lo, hi;  // Eq. 2
            if (amax_b <= e.z) {
                lo = quant8_fast(w, e.x, e.y);
                hi = quant8_fast(w + 4, e.x, e.y);
            } else {
                lo = quant8(w, e.x);
                hi = quant8(w + 4, e.x);
            }
            buf_store8(lo, hi, cs, el >> 1);
            buf_store1(code, ss, el >> 4);
        }
    };
    // two register stages: the next item's loads are in flight while this
    // one is quantized
    for (;;) {
        load_item(it + nw, vb);
        quant_item(it, va);
        it += nw;
        if (it >= items) break;
        load_item(it + nw, va);
        quant_item(it, vb);
        it += nw;
        if (it >= items) break;
    }
}

int64_t quant_items(int64_t rows, int64_t cols) { return rows * (((cols >> 3) + kSeg - 1) / kSeg); }

// Workgroups of the quantize kernel: one per 4 items, at most as many as the
// device holds at once (each wave then loops over items with its loads
// pipelined).
template <bool kDynamic>
int quant_grid(int64_t rows, int64_t cols) {
    static int resident[16] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
    if (resident[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_kernel<kDynamic>, kThreads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 4;
        resident[dev] = cus * per_cu;
    }
    int64_t g = (quant_items(rows, cols) + kWaves - 1) / kWaves;
    if (g > resident[dev]) g = resident[dev];
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
    if (quant_items(rows, cols) >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    dim3 grid(dynamic ? quant_grid<true>(rows, cols) : quant_grid<false>(rows, cols)), block(kThreads);
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
