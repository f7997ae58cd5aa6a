// Output-tile scheduling shared by the GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Logical tile (tm, tn) of workgroup blockIdx.x.  Workgroups are dealt
// round-robin to the 8 XCDs, each with its own L2: consecutive logical tiles
// are given to one XCD, and tiles are walked in groups of 8 tile-rows so the
// W tiles of a group are reused from L2 across its rows.
template <int BM, int BN>
__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int &tm, int &tn) {
    const int num_tm = (int)((M + BM - 1) / BM), num_tn = (int)((N + BN - 1) / BN);
    const int nb = gridDim.x;
    int bid = blockIdx.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    constexpr int G = 8;
    const int per_group = G * num_tn;
    const int group = bid / per_group;
    const int first_tm = group * G;
    const int gsize = min(num_tm - first_tm, G);
    const int in = bid % per_group;
    tm = first_tm + in % gsize;
    tn = in / gsize;
}

// LDS tile rows of 128 bytes (eight 16-byte chunks): chunk c of row r sits in
// slot c ^ f(r).  Measured on gfx950, 16-byte LDS reads are
// served 16 lanes per cycle across 64 banks (two 128-byte rows) and 16-byte
// writes 8 lanes per cycle across 32 banks (one row).  An MFMA operand read
// touches 16 consecutive rows (16-aligned) at one chunk, so f must be one-to-
// one on the even rows and on the odd rows of each 16-row group; a staging
// write touches 4 consecutive rows (4-aligned) at chunks {k, k + 4}, so f's
// low two bits must differ across each 4-row group.  f(r) = s((r >> 1) & 7)
// ^ (r & 1), with s swapping bits 0 and 1, satisfies both.
__device__ __forceinline__ int lds_swz(int row) {
    const int m = (row >> 1) & 7;
    return (((m & 1) << 1) | ((m >> 1) & 1) | (m & 4)) ^ (row & 1);
}
}  // namespace nvfp4
