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

// Tensor-scale source of the quantize pass: static (the caller's alpha), the
// amax pass's partials, or the workgroup's own pass over a small tensor.
enum AlphaSrc { ALPHA_STATIC = 0, ALPHA_PARTIALS = 1, ALPHA_SELF = 2 };

// Max |x| over a whole small tensor (at most kSelfRounds * kSelfLoads *
// kThreads octets) by one workgroup, as FP32 bits of the BF16 maximum: every
// workgroup of the single-launch mode reads the tensor once, in rounds of
// kSelfLoads loads per thread that are all in flight together, instead of
// waiting for a separate amax launch.  Slots past the tensor load its first
// octet again (it is part of the tensor, so the maximum is unchanged): the
// loads of a round carry no condition and are all issued before the first
// use.  The round count is uniform across the workgroup.
constexpr int kSelfLoads = 16;
constexpr int kSelfRounds = 2;
__device__ __forceinline__ uint32_t tensor_amax_bits(const uint16_t *__restrict__ x, uint32_t rows, uint32_t octs,
                                                     int64_t ld) {
    const uint32_t total = rows * octs;
    ushort2_t m = {0, 0};
    for (uint32_t base = 0; base < total; base += kSelfLoads * kThreads) {
        uint4 v[kSelfLoads];
#pragma unroll
        for (int u = 0; u < kSelfLoads; ++u) {
            const uint32_t o = base + threadIdx.x + u * kThreads, oc = o < total ? o : 0u, r = oc / octs;
            v[u] = *reinterpret_cast<const uint4 *>(x + (int64_t)r * ld + (oc - r * octs) * 8);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the round issued before the first use
#pragma unroll
        for (int u = 0; u < kSelfLoads; ++u) {
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].x));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].y));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].z));
            m = __builtin_elementwise_max(m, abs_bf16x2(v[u].w));
        }
    }
    return max((uint32_t)m.x, (uint32_t)m.y) << 16;
}
static_assert(kSelfRounds * kSelfLoads * kThreads * 8 >= kSelfAmaxMaxElems,
              "the single-launch amax reads the whole tensor in at most kSelfRounds rounds");

// Work items of the quantize pass: item it is one wave's (row, segment) of
// kSeg octets; lane l owns whole 16-element blocks, elements
// seg * 2048 + j * 1024 + 16 l .. + 16 for j = 0, 1 (two 16-byte loads each).
// Buffer resources over that row of X, codes and scales (empty past the last
// item) turn out-of-range loads into zeros and drop out-of-range stores,
// without branches.  32-bit item arithmetic: the host guarantees
// items < 2^31 and cols < 2^30.
struct QItems {
    const uint16_t *x;
    uint8_t *codes, *scales;
    int64_t cols, ld;
    uint32_t nseg, items, lane;
    uint32_t pk_bytes;  // kPk: bytes of the packed activation at `codes`

    __device__ __forceinline__ void load(uint32_t it, uint4 *v) const {
        const bool ok = it < items;
        const uint32_t r = ok ? it / nseg : 0u, e0 = (it - r * nseg) * (kSeg * 8) + lane * 16u;
        const rsrc_t xs = make_rsrc(x + (int64_t)r * ld, ok ? (uint32_t)cols * 2u : 0u);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            v[2 * j] = buf_load16(xs, (e0 + 1024u * j) * 2u);
            v[2 * j + 1] = buf_load16(xs, (e0 + 1024u * j) * 2u + 16u);
        }
    }

    // Eq. 3 against t = alpha * 6 (rt = RN(1/t)), Eq. 2 through the divisor
    // table, codes and scale bytes stored: row-major, or (kPk) in the decode
    // kernel's block layout, where block (r / 16, el / 128) holds the 8 code
    // bytes of elements el .. el + 15 of row r at 16 l + (el % 32) / 2 with
    // l = r % 16 + 16 ((el % 128) / 32) (the bytes decode lane l loads), and
    // their scale at 1024 + 8 (r % 16) + (el % 128) / 16
    template <bool kPk>
    __device__ __forceinline__ void quant(uint32_t it, const uint4 *v, float t, float rt, const float4 *dtab) const {
        const bool ok = it < items;
        const uint32_t r = ok ? it / nseg : 0u, e0 = (it - r * nseg) * (kSeg * 8) + lane * 16u;
        const rsrc_t cs = kPk ? make_rsrc(codes, pk_bytes)
                              : make_rsrc(codes + (int64_t)r * (cols >> 1), ok ? (uint32_t)(cols >> 1) : 0u);
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
            if constexpr (kPk) {
                const uint32_t blk = ((r >> 4) * (uint32_t)(cols >> 7) + (el >> 7)) * (uint32_t)kPackBlock;
                const bool in = ok & (el < (uint32_t)cols);
                const uint32_t co = blk + 16u * ((r & 15u) + 16u * ((el & 127u) >> 5)) + ((el & 31u) >> 1);
                const uint32_t so = blk + 1024u + 8u * (r & 15u) + ((el & 127u) >> 4);
                buf_store8(lo, hi, cs, in ? co : kBufOOB);
                buf_store1(code, cs, in ? so : kBufOOB);
            } else {
                buf_store8(lo, hi, cs, el >> 1);
                buf_store1(code, ss, el >> 4);
            }
        }
    }
};

// Per E4M3 scale code: the divisor d = fl32(alpha * sigma), RN(1/d), and
// the largest |x| the fast path of quant8_fast takes (-1 when d is outside
// [2^-90, 2^100], zero included, so those blocks take quant8); threads 0-127
// fill one entry each, the caller's LDS barrier follows.
__device__ __forceinline__ void fill_dtab(float4 *dtab, float alpha) {
    if (threadIdx.x < 128) {
        const float d = alpha * e4m3_decode(threadIdx.x);
        const bool in = d >= 0x1p-90f && d <= 0x1p100f;
        dtab[threadIdx.x] = make_float4(d, in ? div_rn(1.0f, d) : 0.0f, in ? d * 0x1p120f : -1.0f, 0.0f);
    }
}

template <int kAlpha, bool kPk = false>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld, uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales, float *__restrict__ alpha_io,
                                                            const uint32_t *__restrict__ partials, int nparts,
                                                            uint32_t pk_bytes) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // 32-bit item arithmetic: the host guarantees items < 2^31 and cols < 2^30
    const uint32_t octs = (uint32_t)(cols >> 3);  // 8-element groups per row; even, so pairs never straddle rows
    const uint32_t nseg = (octs + kSeg - 1) / kSeg;
    const uint32_t items = (uint32_t)rows * nseg, nw = gridDim.x * kWaves;
    const QItems qi{x, codes, scales, cols, ld, nseg, items, lane, pk_bytes};
    uint32_t it = blockIdx.x * kWaves + wave;
    // the tensor scale's inputs are read first, then the first item's loads
    // are issued, so waiting for the former leaves the latter in flight
    // (nparts <= kMaxParts: at most kMaxParts / kThreads partials per thread,
    // loaded without branches; entries past nparts read as zero)
    constexpr int kPartsPerThread = kMaxParts / kThreads;
    uint32_t pv[kPartsPerThread];
    if (kAlpha == ALPHA_PARTIALS) {
        const rsrc_t ps = make_rsrc(partials, (uint32_t)nparts * 4u);
#pragma unroll
        for (int j = 0; j < kPartsPerThread; ++j)
            pv[j] = __builtin_amdgcn_raw_buffer_load_b32(ps, (threadIdx.x + j * kThreads) * 4u, 0, 0);
    }
    const float alpha_in = kAlpha == ALPHA_STATIC ? *alpha_io : 0.0f;
    asm volatile("" ::: "memory");
    uint4 va[2 * kBlk], vb[2 * kBlk];
    qi.load(it, va);
    float alpha = alpha_in;
    if (kAlpha != ALPHA_STATIC) {
        uint32_t pmax = 0;
        if constexpr (kAlpha == ALPHA_PARTIALS) {
#pragma unroll
            for (int j = 0; j < kPartsPerThread; ++j) pmax = max(pmax, pv[j]);
        } else {
            pmax = tensor_amax_bits(x, (uint32_t)rows, octs, ld);
        }
        alpha = alpha_from_max(pmax);
        if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_io = alpha;
    }
    const float t = alpha * kQmax;
    const float rt = t > 0.0f ? div_rn(1.0f, t) : 0.0f;
    __shared__ float4 dtab[128];
    fill_dtab(dtab, alpha);
    lds_barrier();
    // two register stages: the next item's loads are in flight while this
    // one is quantized
    for (;;) {
        qi.load(it + nw, vb);
        qi.quant<kPk>(it, va, t, rt, dtab);
        it += nw;
        if (it >= items) break;
        qi.load(it + nw, va);
        qi.quant<kPk>(it, vb, t, rt, dtab);
        it += nw;
        if (it >= items) break;
    }
}

int64_t quant_items(int64_t rows, int64_t cols) { return rows * (((cols >> 3) + kSeg - 1) / kSeg); }

// Workgroups of the quantize kernel: one per 4 items, at most as many as the
// device holds at once (each wave then loops over items with its loads
// pipelined).
// The per-device count is cached in an atomic: threads that race on the first
// call compute the same value and store it, so no lock is needed.
template <int kAlpha>
int quant_grid(int64_t rows, int64_t cols) {
    static std::atomic<int> resident_cache[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int resident = dev < 16 ? resident_cache[dev].load(std::memory_order_relaxed) : 0;
    if (resident == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quantize_kernel<kAlpha>, kThreads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 4;
        resident = cus * per_cu;
        if (dev < 16) resident_cache[dev].store(resident, std::memory_order_relaxed);
    }
    int64_t g = (quant_items(rows, cols) + kWaves - 1) / kWaves;
    if (g > resident) g = resident;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace

// Scratch of the allocation-free entry point (nvfp4_quantize_noalloc): the
// dynamic tensor scale's per-workgroup partial maxima, at most kMaxParts of
// them (4 KB).  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it.  The partials need no
// clearing: the amax pass writes each entry the quantize pass reads.
static __device__ __align__(256) uint32_t scratch[kMaxParts];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.  Host code never passes `scratch` itself
// to a kernel: its host-side name is a stand-in, not a device address.
hipError_t quantize_scratch(uint32_t **ptr, size_t *bytes) {
    constexpr int kDevs = 64;
    static std::atomic<uint32_t *> cache[kDevs];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    uint32_t *p = dev >= 0 && dev < kDevs ? cache[dev].load(std::memory_order_acquire) : nullptr;
    if (!p) {
        e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        if (dev >= 0 && dev < kDevs) cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    *bytes = sizeof(scratch);
    return hipSuccess;
}

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

bool quantize_self_amax(int64_t rows, int64_t cols) { return rows * cols <= kSelfAmaxMaxElems; }

hipError_t launch_quantize_dynamic(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                                   uint8_t *scales, float *alpha, uint32_t *partials, int nparts, hipStream_t s,
                                   bool pack_a) {
    if (quant_items(rows, cols) >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    if (!quantize_self_amax(rows, cols))
        if (hipError_t e = launch_amax_partials(x, rows, cols, ld, partials, nparts, s); e != hipSuccess) return e;
    return launch_quantize(x, rows, cols, ld, codes, scales, alpha, 1, partials, nparts, s, pack_a);
}

namespace {

template <bool kPk>
void launch_quantize_kind(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes, uint8_t *scales,
                          float *alpha, int dynamic, const uint32_t *partials, int nparts, hipStream_t s,
                          uint32_t pk_bytes) {
    const dim3 block(kThreads);
    if (dynamic && quantize_self_amax(rows, cols))
        hipLaunchKernelGGL((quantize_kernel<ALPHA_SELF, kPk>), dim3(quant_grid<ALPHA_SELF>(rows, cols)), block, 0, s,
                           x, rows, cols, ld, codes, scales, alpha, partials, nparts, pk_bytes);
    else if (dynamic)
        hipLaunchKernelGGL((quantize_kernel<ALPHA_PARTIALS, kPk>), dim3(quant_grid<ALPHA_PARTIALS>(rows, cols)), block,
                           0, s, x, rows, cols, ld, codes, scales, alpha, partials, nparts, pk_bytes);
    else
        hipLaunchKernelGGL((quantize_kernel<ALPHA_STATIC, kPk>), dim3(quant_grid<ALPHA_STATIC>(rows, cols)), block, 0,
                           s, x, rows, cols, ld, codes, scales, alpha, partials, nparts, pk_bytes);
}

}  // namespace

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                           uint8_t *scales, float *alpha, int dynamic, const uint32_t *partials, int nparts,
                           hipStream_t s, bool pack_a) {
    if (quant_items(rows, cols) >= (int64_t(1) << 31) || cols >= (int64_t(1) << 30)) return hipErrorInvalidValue;
    if (pack_a) {
        const size_t pk = decode_pack_a_bytes(rows, cols);
        if (cols % 128 != 0 || pk >= (size_t(1) << 31)) return hipErrorInvalidValue;
        launch_quantize_kind<true>(x, rows, cols, ld, codes, scales, alpha, dynamic, partials, nparts, s,
                                   (uint32_t)pk);
    } else {
        launch_quantize_kind<false>(x, rows, cols, ld, codes, scales, alpha, dynamic, partials, nparts, s, 0u);
    }
    return hipGetLastError();
}

namespace {

// Eq. 3 / Eq. 2 on FP32 values, each taken as it is (a GEMM output quantized
// for the next layer): one 16-element block per lane and iteration, the tensor
// scale read from device memory.  Eq. 3: s = RN(amax / t), t = RN(alpha * 6),
// by Markstein's correction against one reciprocal of t where that is exact
// (t in [2^-100, 2^100], amax zero or in [2^-100, t * 2^120]), else the IEEE
// quotient; the hardware FP32 -> FP8 convert after the clamp to 448.  Eq. 2:
// d = RN(alpha * sigma), each element's RN(y / d) by the corrected quotient
// against RN(1/d) under the same conditions (and no nonzero |y| below
// 2^-100), else the IEEE quotient; d == 0 gives signed zeros.  E2M1 by the
// hardware FP32 -> FP4 convert (nearest-even, saturating, sign kept).
__global__ __launch_bounds__(kThreads) void quantize_f32_kernel(const float *__restrict__ y, int64_t rows,
                                                                int64_t cols, int64_t ld, uint8_t *__restrict__ codes,
                                                                uint8_t *__restrict__ scales,
                                                                const float *__restrict__ alpha) {
    const float ya = *alpha;
    const float t6 = ya * kQmax, rt6 = t6 > 0.0f ? div_rn(1.0f, t6) : 0.0f;
    const bool tfast = (t6 >= 0x1p-100f) & (t6 <= 0x1p100f);
    const int64_t bpr = cols >> 4, nblk = rows * bpr;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * kThreads) {
        const int64_t r = b / bpr, c = b - r * bpr;
        const float4 *p = reinterpret_cast<const float4 *>(y + r * ld + c * 16);
        float v[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float4 t = p[e];
            v[4 * e] = t.x;
            v[4 * e + 1] = t.y;
            v[4 * e + 2] = t.z;
            v[4 * e + 3] = t.w;
        }
        uint32_t am = 0;
        bool tiny = false;  // a nonzero |y| below 2^-100
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t ab = __float_as_uint(v[e]) & 0x7FFFFFFFu;
            am = max(am, ab);
            tiny = tiny | ((ab != 0u) & (ab < 0x0D800000u));
        }
        const float amax = __uint_as_float(am);
        float sq;
        if (tfast & (amax <= t6 * 0x1p120f) & ((amax == 0.0f) | (amax >= 0x1p-100f))) {
            const float q0 = amax * rt6;
            sq = __builtin_fmaf(__builtin_fmaf(-q0, t6, amax), rt6, q0);
        } else {
            sq = t6 > 0.0f ? div_rn(amax, t6) : 0.0f;
        }
        const uint32_t code = e4m3_encode(sq);
        const float d = ya * e4m3_decode(code);
        const float rd = d > 0.0f ? div_rn(1.0f, d) : 0.0f;
        float qv[16];
        if ((d >= 0x1p-100f) & (d <= 0x1p100f) & !tiny & (amax <= d * 0x1p120f)) {
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
        uint32_t w0 = 0, w1 = 0;
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[0], qv[1], 1.0f, 0);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[2], qv[3], 1.0f, 1);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[4], qv[5], 1.0f, 2);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, qv[6], qv[7], 1.0f, 3);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[8], qv[9], 1.0f, 0);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[10], qv[11], 1.0f, 1);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[12], qv[13], 1.0f, 2);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, qv[14], qv[15], 1.0f, 3);
        uint32_t *cp = reinterpret_cast<uint32_t *>(codes + r * (cols >> 1) + c * 8);
        cp[0] = w0;
        cp[1] = w1;
        scales[r * bpr + c] = (uint8_t)code;
    }
}

}  // namespace

hipError_t launch_quantize_f32(const float *y, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                               uint8_t *scales, const float *alpha, hipStream_t s) {
    const int64_t nblk = rows * (cols >> 4);
    if (nblk <= 0) return hipSuccess;
    int64_t g = (nblk + kThreads - 1) / kThreads;
    if (g > 16384) g = 16384;
    hipLaunchKernelGGL(quantize_f32_kernel, dim3((unsigned)g), dim3(kThreads), 0, s, y, rows, cols, ld, codes, scales,
                       alpha);
    return hipGetLastError();
}

hipError_t launch_alpha_from_partials(const uint32_t *partials, int nparts, float *alpha, hipStream_t s) {
    hipLaunchKernelGGL(alpha_kernel, dim3(1), dim3(kThreads), 0, s, partials, nparts, alpha);
    return hipGetLastError();
}

}  // namespace nvfp4
