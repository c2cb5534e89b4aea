// Device-side helpers shared by the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Compute units and XCDs of an MI355X.  Workgroups are handed to the XCDs
// round-robin (workgroup id modulo 8), and every XCD has its own L2.
constexpr int kNumXcd = 8;

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Pack the low halves / high halves of two dwords: lo16(x) | lo16(y) << 16
// and hi16(x) | hi16(y) << 16.  Used to transpose 2-byte elements in registers.
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
    return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
    return (x >> 16) | (y & 0xffff0000u);
}

// Map a linear workgroup id to an output tile (tm, tn).
//
// 1. XCD-aware remap: workgroups are dealt to the eight XCDs in round-robin
//    order, so ids equal modulo 8 share an XCD.  Consecutive "virtual"
//    ids v are given to one such class, so a run of neighbouring tiles shares that
//    XCD's L2 instead of being spread over all eight.
// 2. Grouped order: tiles are walked column by column inside bands of
//    group_m tile-rows, so the workgroups resident at one time reuse a few
//    A row-panels and B column-panels from L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    const int full = nwg - (nwg % kNumXcd);
    return bid < full ? (bid % kNumXcd) * (full / kNumXcd) + bid / kNumXcd : bid;
}

__device__ __forceinline__ void grouped_tile(int v, int tiles_m, int tiles_n, int group_m,
                                             int &tm, int &tn) {
    const int group_size = group_m * tiles_n;
    const int g = v / group_size;
    const int first_m = g * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int r = v - g * group_size;
    tm = first_m + r % rows;
    tn = r / rows;
}

__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n,
                                            int group_m, int &tm, int &tn) {
    grouped_tile(xcd_remap(bid, nwg), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace mgemm
