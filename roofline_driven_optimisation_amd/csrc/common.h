// Device-side helpers shared by the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

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

// ---- fused Linear-layer epilogue: y = act(x + bias[col]) ------------------
// x is alpha * acc (+ beta * C) in fp32.  The activations are written to be
// short, because a kernel applies them to every output element:
//   * GELU, x * Phi(x): Phi from the rational approximation of erf in
//     Abramowitz and Stegun, Handbook of Mathematical Functions, formula
//     7.1.26 (|error| <= 1.5e-7 in erf), used in its complementary form
//     (0.5 erfc(|x| / sqrt 2) = Phi(-|x|)) so that negative x suffers no
//     cancellation; an error e in Phi moves the output by |x| e;
//   * SiLU, x / (1 + e^-x), with the hardware base-2 exponential and
//     reciprocal (relative errors of a few 1e-7, growing with |x| through
//     the rounding of -x log2(e));
//   * ReLU, 0 for x < 0 (NaN passes through).
__device__ __forceinline__ float phi_neg_abs(float x) {  // Phi(-|x|)
    const float y = fabsf(x) * 0.70710678118654752f;      // |x| / sqrt 2
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, y, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    return 0.5f * (p * t) * __expf(-y * y);
}
template <int ACT>
__device__ __forceinline__ float activate_t(float x) {
    if constexpr (ACT == kActRelu) {
        return x < 0.0f ? 0.0f : x;
    } else if constexpr (ACT == kActGelu) {
        const float q = phi_neg_abs(x);
        return x * (x < 0.0f ? q : 1.0f - q);
    } else if constexpr (ACT == kActSilu) {
        return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
    } else {
        return x;
    }
}
__device__ __forceinline__ float activate(float x, int act) {
    switch (act) {
        case kActRelu: return activate_t<kActRelu>(x);
        case kActGelu: return activate_t<kActGelu>(x);
        case kActSilu: return activate_t<kActSilu>(x);
        default: return x;
    }
}
// Calls f(std::integral_constant<int, act>()), so that a loop can be compiled
// once per activation instead of switching per element.
template <class F>
__device__ __forceinline__ void with_activation(int act, F &&f) {
    switch (act) {
        case kActRelu: f(std::integral_constant<int, kActRelu>()); break;
        case kActGelu: f(std::integral_constant<int, kActGelu>()); break;
        case kActSilu: f(std::integral_constant<int, kActSilu>()); break;
        default: f(std::integral_constant<int, kActNone>()); break;
    }
}
// The bias of columns col .. col + 3 (bias points at column 0 of the range
// the caller addresses; zero at or past `cols` or without a bias).
template <bool EPI>
__device__ __forceinline__ f32x4 bias4(const float *bias, int col, int cols) {
    f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (EPI) {
        if (bias != nullptr) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < cols) b[e] = bias[col + e];
        }
    }
    return b;
}
template <bool EPI>
__device__ __forceinline__ float epi_apply(float x, float b, int act) {
    if constexpr (EPI)
        return activate(x + b, act);
    else
        return x;
}

// Pack the low halves / high halves of two dwords: lo16(x) | lo16(y) << 16
// and hi16(x) | hi16(y) << 16.  Used to transpose 2-byte elements in registers.
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
    return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
    return (x >> 16) | (y & 0xffff0000u);
}

// ---- raw buffer descriptors and direct global -> LDS copies ---------------
// An offset past every descriptor range (all ranges are clamped below 2^31).
// Buffer builtins take the offset as int: always pass static_cast<int>(...).
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

// The same raw-buffer descriptor as four dwords (base, stride 0, range, flags).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_desc(const void *base, long long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4 d;
    d.x = static_cast<int>(static_cast<uint32_t>(p));
    d.y = static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu);
    d.z = static_cast<int>(bytes);
    d.w = kRsrcFlags;
    return d;
}

// One direct global -> LDS copy: 16 bytes per lane from byte offset `voff`
// of the buffer `desc` into LDS at `lds_addr` + 16 * lane.  sc0 makes the
// load bypass the vector L1 (the data is used once per workgroup and lands
// in LDS; about 4% faster on the square bf16 GEMM than a cached load).  Written as inline
// assembly on purpose: the compiler then does not model it as an LDS write
// and does not stall the fragment reads of the other stage behind it (it
// cannot prove the two stages apart); the K loop waits for these copies
// explicitly (s_waitcnt + barrier) before reading the stage they fill.  M0
// holds the LDS address for the instruction and is restored afterwards; the
// s_nop is the wait state required between an M0 write and an LDS DMA.
__device__ __forceinline__ void lds_dma16(i32x4 desc, uint32_t lds_addr, uint32_t voff) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen sc0 lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(desc)
        : "memory");
}

// An L2 warm-up load with no register destination: 4 bytes per lane from
// byte offset `voff` of `desc` into LDS at `lds_addr` + 4 * lane (a scratch
// area nothing reads).  Without sc0 the line is kept in L2 for the copy
// that follows it; like lds_dma16 it is waited for only through the
// vector-memory counter, never by the compiler.
__device__ __forceinline__ void lds_dma4_warm(i32x4 desc, uint32_t lds_addr, uint32_t voff) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(desc)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p));
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
