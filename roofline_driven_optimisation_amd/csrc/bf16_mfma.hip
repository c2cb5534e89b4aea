// bf16-input, fp32-accumulate GEMM on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), LDS-tiled and multi-buffered.  Three kernels:
//   * bf16_mfma_kernel: four waves, one per SIMD, K step 64, two LDS stages;
//     each wave interleaves its LDS reads with its own MFMAs (the 256 x 128,
//     128 x 256 and 128 x 128 tiles);
//   * bf16_q4_kernel (further down): the 256 x 256 four-wave tile, K step
//     32, four LDS stages filled three steps ahead;
//   * bf16_pp_kernel (further down): eight waves, two per SIMD, K step 32,
//     four LDS stages; the two waves of a SIMD take turns reading fragments
//     and running MFMAs (ping-pong), so MFMAs do not wait on LDS reads.
// The tile picker at the end chooses between them by shape.
//
// Last-round split (both 256 x 256 kernels and the 8-bit float kernel).  A
// 256 x 256 tile count that leaves a last round at most half full (2048 x
// 4096: 128 tiles; 2048 x 12288: 384 on 256 CUs) wastes up to half of that
// round.  Its r tiles are then computed by 2 r workgroups, each over part of
// the K steps: the first of a pair to start posts its fp32 partial tile and
// publishes it (release store of an epoch number the host chose for the
// call); the second waits for it (acquire) and writes alpha * (own +
// partial) + beta * C.  Roles are decided when the workgroups start (an
// atomic swap on the tile's claim word: the first to claim posts), so a
// workgroup only waits for one that is already running and never waits
// itself, and the wait ends whatever order the hardware dispatched the
// workgroups in; the sum of two partials does not depend on the order in
// which they are added.  When r is a multiple of 8 the pair is
// workgroups b and b + 8, which the hardware places on the same XCD, and the
// partial goes through that XCD's L2 in ordinary memory; otherwise the pair
// is 2i and 2i + 1, on different XCDs, and the partial goes through uncached
// memory.  The pages do not cover this; it is the split-K idea applied to
// the wave-quantisation loss they discuss for small grids.
//
// Structure of the four-wave kernel (page "Naive GEMM and Roofline
// analysis", section 10.4, the three tile levels plus double buffering):
//   * workgroup tile BM x BN (256 or 128 each), K step 64, 256 threads = four
//     64-lane waves in 2 x 2, each owning a (BM/2) x (BN/2) sub-tile built from
//     32 x 32 MFMA blocks; a 128 x 128 wave tile keeps 256 fp32 accumulators
//     per lane (the whole AccVGPR file), which is what keeps the LDS bytes per
//     MFMA low enough for the LDS to keep up;
//   * global -> LDS copies use buffer_load ... lds: each lane's 16 bytes go
//     straight into LDS at M0 + 16 * lane, with no staging registers and no
//     LDS write instructions.  Tile k+1 is requested into the other LDS buffer
//     before tile k's MFMAs start and is waited for after they finish (page
//     "Where kernel performance comes from", overlap section: load k+1 while
//     computing k), so one barrier per K step suffices;
//   * MFMA operand fragments are double-buffered in registers: the reads for
//     k16 sub-step s+1 are issued before the MFMAs of sub-step s;
//   * fused alpha/beta epilogue in fp32 with 16-byte stores (the MFMAs compute
//     transposed blocks, see store_c_tile); C is not read when beta == 0.
//
// Edges.  The buffer resource's range check turns every out-of-range load
// into zeros and drops every out-of-range store; a column or k index past the
// matrix (which would otherwise wrap into the next row) is redirected to an
// out-of-range offset.  The main loop has no branches on the shape.
//
// Operand layouts in LDS.  The gfx950 LDS serves 256 bytes per clock (64
// four-byte banks): a 16-byte-per-lane read is served 16 lanes per clock and
// an 8-byte-per-lane read 32 lanes per clock, and each such lane group must
// touch 64 distinct banks to run at full rate.  Rows are stored as 16-byte
// chunks, XOR-swizzled (the software form of the swizzled layouts of page
// "Memory hierarchy and cost table", section 4.3.4):
//   * A tile: BM rows of 64 k (128 bytes, 8 chunks); chunk c of row r sits at
//     position c ^ ((r / 2) % 8).  A fragment (row l % 32, k-octet l / 32) is
//     one ds_read_b128; 16 consecutive rows share one chunk index, fall into
//     two 128-byte halves of a bank line by parity and into 8 positions by
//     the key, so every 16-lane group covers the 64 banks once.
//   * B tile: 64 k-rows of BN n (natural row-major, 256 or 512 bytes);
//     chunk c of row k sits at position c ^ swz_b(k).  The B fragment needs 8
//     k-consecutive values of one column per lane; ds_read_b64_tr_b16
//     provides that transpose: within a 16-lane group, lane i receives
//     element i % 4 of the 8 bytes read by lanes 4e + i / 4 (e = 0..3).  So
//     if lane j reads the 4 columns n0 + 4 (j % 4) .. +3 of row k0 + j / 4,
//     lane i gets rows k0 .. k0+3 of column n0 + i; two such reads give the 8
//     k values of a fragment.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

// s_waitcnt immediate that waits until at most `vm` vector-memory operations
// are outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima).
constexpr int wait_vm(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;    // wave tile
    static constexpr int MI = WM / 32, NI = WN / 32;  // 32 x 32 MFMA blocks per wave
    static constexpr int A_LOADS = BM / 32;           // 1 KB wave-loads of A per wave per K step
    static constexpr int B_CHUNKS = BN / 8;           // 16-byte chunks per B row
    static constexpr int B_ROWS_PER_LOAD = 64 / B_CHUNKS;
    static constexpr int B_LOADS = BN / 32;           // 1 KB wave-loads of B per wave per K step
    static constexpr int A_STAGE = BM * kBK;          // bf16 elements per stage
    static constexpr int B_STAGE = kBK * BN;
};

// Swizzle key of B row k (XOR on chunk-index bits 2..3, i.e. on 64-byte
// segments).  A 32-lane half of a transposed read covers 4 consecutive rows x
// one aligned 64-byte segment; the key sends the 4 rows to the 4 different
// 64-byte quarters of a 256-byte bank line.  It depends on k % 4 only, so a
// lane's read address changes by plain immediate offsets across rows and k16
// sub-steps.
__device__ __forceinline__ int swz_b(int k) { return (k & 3) << 2; }

// Swizzle key of A row r (see the layout notes above).
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }

// Epilogue of one wave: C = alpha * acc + beta * C for MI x NI blocks of 32 x
// 32.  The MFMAs take the B fragment as their first operand and the A
// fragment as their second, so each block holds the transposed product: in
// register r of lane l sits C[row l % 32][column 8 (r / 4) + 4 (l / 32) +
// r % 4] of the block, i.e. registers 4 g .. 4 g + 3 are four consecutive
// columns, written (and, with beta != 0, read) as one 16-byte access.  The
// descriptor `rc` is based at the workgroup tile origin and ends at the last
// element of C, so rows past M fall outside it; a 4-column group past N
// (N is a multiple of 8, so a group is entirely inside or outside) is
// redirected out of range.  Stores of one block are issued before the next
// block is converted, which bounds the registers in use.  With EPI the fused
// epilogue follows alpha/beta: act(x + bias[col]), `bias` based at the tile's
// first column.
template <int MI, int NI, bool EPI = false>
__device__ __forceinline__ void store_c_tile(const f32x16 (&acc)[MI][NI],
                                             __amdgpu_buffer_rsrc_t rc, int row0, int col0,
                                             int cols_left, int N, float alpha, float beta,
                                             const float *bias = nullptr, int act = kActNone) {
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, h = lane >> 5;
    const bool read_c = beta != 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int row = row0 + 32 * i + l32;
        auto offset = [&](int jj, int g) {
            const int col = col0 + 32 * jj + 8 * g + 4 * h;
            return col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
        };
        // The block row's C loads are all issued before its stores: the
        // compiler cannot tell loads and stores of C apart, so a load placed
        // after a store would wait for it.
        f32x4 cin[NI][4];
        if (read_c) {
#pragma unroll
            for (int jj = 0; jj < NI; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    cin[jj][g] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rc, static_cast<int>(offset(jj, g)), 0, 0));
        }
#pragma unroll
        for (int jj = 0; jj < NI; ++jj) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = alpha * acc[i][jj][4 * g + e];
                if (read_c) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, cin[jj][g][e], out[e]);
                }
                if constexpr (EPI) {
                    const f32x4 bv = bias4<EPI>(bias, col0 + 32 * jj + 8 * g + 4 * h, cols_left);
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = epi_apply<EPI>(out[e], bv[e], act);
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rc,
                                                       static_cast<int>(offset(jj, g)), 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Epilogue through LDS for a wave tile 64 columns wide: the wave writes 64
// rows of its tile into a private 16 KB LDS region (16-byte chunk c of row r
// at position c ^ (r % 16), so the 16 lanes served together hit 64 distinct
// banks both when writing and when reading back), reads them back row by
// row and stores them with 16 lanes per 256-byte row segment, four rows per
// instruction: every store instruction covers 8 whole 128-byte lines instead
// of 32 partial ones.  Same semantics and edge handling as store_c_tile.
// Modes: kStoreC writes alpha * acc (+ beta * C); kPostPartial writes the raw
// accumulators to a BM x BN row-major partial tile `rw` (ldw floats per row)
// and never touches C; kAddPartial writes alpha * (acc + partial) (+ beta *
// C).  PLOAD is the cache policy of the partial loads: system scope (sc0
// sc1) when the partial was written on another XCD, device scope (sc1: past
// the CU's L1, served by the XCD's L2) when it was written on the same XCD.
enum EpilogueMode { kStoreC, kPostPartial, kAddPartial };
constexpr int kSystemScope = 1 | 16;  // buffer cache policy sc0 sc1: no stale L1 / L2 copy
constexpr int kDeviceScope = 16;      // buffer cache policy sc1: no stale L1 copy

template <int MI, int NI, EpilogueMode MODE, int PLOAD = kSystemScope, bool EPI = false>
__device__ __forceinline__ void store_c_tile_lds(const f32x16 (&acc)[MI][NI], float *region,
                                                 __amdgpu_buffer_rsrc_t rc, int row0, int col0,
                                                 int cols_left, int N, float alpha, float beta,
                                                 __amdgpu_buffer_rsrc_t rw, int ldw,
                                                 const float *bias = nullptr,
                                                 int act = kActNone) {
    static_assert(NI * 32 == 64 && MI % 2 == 0, "wave tile must be (64 k) x 64");
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, h = lane >> 5;
    const bool read_c = beta != 0.0f;
    // the lane's four columns are the same in both halves: bias loaded once,
    // before any store
    const f32x4 bv = bias4<EPI && MODE != kPostPartial>(bias, col0 + 4 * (lane & 15), cols_left);
#pragma unroll
    for (int half = 0; half < MI / 2; ++half) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            const int r = 32 * i2 + l32;
#pragma unroll
            for (int jj = 0; jj < NI; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int chunk = 8 * jj + 2 * g + h;
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[2 * half + i2][jj][4 * g + e];
                    *reinterpret_cast<f32x4 *>(&region[r * 64 + ((chunk ^ (r & 15)) * 4)]) = v;
                }
        }
        const int chunk = lane & 15;
        const int col = col0 + 4 * chunk;
        // Rows in groups of kGroup: the group's global loads (partial, C)
        // are all issued before its stores.  The compiler cannot tell the
        // loaded buffers from the stored C apart, so a load placed after a
        // store would wait for it: one memory round trip per row.
        constexpr int kGroup = 8;
#pragma unroll
        for (int j0 = 0; j0 < 16; j0 += kGroup) {
            f32x4 pv[kGroup], cv[kGroup];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int r = 4 * (j0 + u) + (lane >> 4);
                const int row = row0 + 64 * half + r;
                if (MODE == kAddPartial)
                    pv[u] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rw, ((row * ldw) + col0 + 4 * chunk) * 4, 0, PLOAD));
                if (MODE != kPostPartial && read_c) {
                    const uint32_t off =
                        col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                    cv[u] = __builtin_bit_cast(
                        f32x4,
                        __builtin_amdgcn_raw_buffer_load_b128(rc, static_cast<int>(off), 0, 0));
                }
            }
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int r = 4 * (j0 + u) + (lane >> 4);
                const f32x4 v =
                    *reinterpret_cast<const f32x4 *>(&region[r * 64 + ((chunk ^ (r & 15)) * 4)]);
                const int row = row0 + 64 * half + r;
                if (MODE == kPostPartial) {
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, v), rw, ((row * ldw) + col0 + 4 * chunk) * 4,
                        0, 0);
                    continue;
                }
                const uint32_t off =
                    col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = alpha * (MODE == kAddPartial ? v[e] + pv[u][e] : v[e]);
                if (read_c) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, cv[u][e], out[e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = epi_apply<EPI>(out[e], bv[e], act);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rc,
                                                       static_cast<int>(off), 0, 0);
            }
        }
    }
}

// Epilogue through LDS for a wave tile 128 columns wide, 32 rows (a band)
// at a time: write_band(i, region) puts band i of the wave's fp32 values into
// a private 16 KB LDS region (16-byte chunk c of row r at position c ^ (r %
// 16), so the 16 lanes served together hit 64 distinct banks both when
// writing and when reading back); the band is read back two rows per
// instruction and stored with 32 lanes per 512-byte row segment: each store
// instruction covers 8 whole 128-byte lines.  C = alpha * acc (+ beta * C);
// same edge handling as store_c_tile.  MODE and PLOAD as for
// store_c_tile_lds (a partial tile `rw` of ldw floats per row).
template <int BANDS, EpilogueMode MODE = kStoreC, int PLOAD = kSystemScope, bool EPI = false,
          class WriteBand>
__device__ __forceinline__ void store_c_bands_lds128(WriteBand &&write_band, float *region,
                                                     __amdgpu_buffer_rsrc_t rc, int row0,
                                                     int col0, int cols_left, int N, float alpha,
                                                     float beta, __amdgpu_buffer_rsrc_t rw,
                                                     int ldw, const float *bias = nullptr,
                                                     int act = kActNone) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const bool read_c = beta != 0.0f;
    // a lane stores the same four columns in every pass: their bias is
    // loaded once, before any store (a load after a store to C would wait)
    const f32x4 bv = bias4<EPI && MODE != kPostPartial>(bias, col0 + 4 * (lane & 31), cols_left);
#pragma unroll
    for (int i = 0; i < BANDS; ++i) {
        write_band(i, region);
        const int chunk = lane & 31;
        const int col = col0 + 4 * chunk;
        // The rows' global loads (partial, C) are issued a group at a time
        // (all 16 rows) before the group's stores: the compiler cannot tell
        // the loaded buffers from the stored C apart, so a load placed after
        // a store would wait for it.
        // With the fused epilogue the combined values go back to the same
        // LDS slots, and a rolled loop applies bias and activation and stores
        // them: one copy of the activation code instead of 64 (fully
        // unrolled, they made the compiler keep the accumulators in scratch).
        constexpr int kGroup = 16;
#pragma unroll
        for (int j0 = 0; j0 < 16; j0 += kGroup) {
            f32x4 pv[kGroup], cv[kGroup];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int row = row0 + 32 * i + 2 * (j0 + u) + h;
                if (MODE == kAddPartial)
                    pv[u] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (row * ldw + col) * 4, 0,
                                                                     PLOAD));
                if (MODE != kPostPartial && read_c) {
                    const uint32_t off =
                        col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                    cv[u] = __builtin_bit_cast(
                        f32x4,
                        __builtin_amdgcn_raw_buffer_load_b128(rc, static_cast<int>(off), 0, 0));
                }
            }
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int r = 2 * (j0 + u) + h;
                f32x4 *slot = reinterpret_cast<f32x4 *>(&region[r * 128 + ((chunk ^ (r & 15)) * 4)]);
                const f32x4 v = *slot;
                const int row = row0 + 32 * i + r;
                if (MODE == kPostPartial) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rw,
                                                           (row * ldw + col) * 4, 0, 0);
                    continue;
                }
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = alpha * (MODE == kAddPartial ? v[e] + pv[u][e] : v[e]);
                if (read_c) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, cv[u][e], out[e]);
                }
                if (EPI) {
                    *slot = out;
                    continue;
                }
                const uint32_t off =
                    col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rc,
                                                       static_cast<int>(off), 0, 0);
            }
        }
        if constexpr (EPI && MODE != kPostPartial) {
            // four rows per iteration: their LDS reads are in flight together
            with_activation(act, [&](auto act_tag) {
                constexpr int ACT = decltype(act_tag)::value;
#pragma unroll 1
                for (int j0 = 0; j0 < 16; j0 += 4) {
                    f32x4 o[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 2 * (j0 + u) + h;
                        o[u] = *reinterpret_cast<const f32x4 *>(
                            &region[r * 128 + ((chunk ^ (r & 15)) * 4)]);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[u][e] = activate_t<ACT>(o[u][e] + bv[e]);
                        const int row = row0 + 32 * i + 2 * (j0 + u) + h;
                        const uint32_t off =
                            col < cols_left ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[u]), rc,
                                                               static_cast<int>(off), 0, 0);
                    }
                }
            });
        }
    }
}

// Band i of a wave's MI x 4 blocks of 32 x 32 (the transposed layout of
// store_c_tile): register 4 g + e of lane l holds row l % 32, column 32 jj +
// 8 g + 4 (l / 32) + e of block (i, jj), i.e. 16-byte chunk 8 jj + 2 g + l / 32.
template <int MI>
__device__ __forceinline__ auto band_writer32(const f32x16 (&acc)[MI][4]) {
    return [&acc](int i, float *region) {
        const int lane = threadIdx.x & 63;
        const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int chunk = 8 * jj + 2 * g + h;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][jj][4 * g + e];
                *reinterpret_cast<f32x4 *>(&region[l32 * 128 + ((chunk ^ (l32 & 15)) * 4)]) = v;
            }
    };
}

template <int MI, EpilogueMode MODE = kStoreC, int PLOAD = kSystemScope, bool EPI = false>
__device__ __forceinline__ void store_c_tile_lds128(const f32x16 (&acc)[MI][4], float *region,
                                                    __amdgpu_buffer_rsrc_t rc, int row0,
                                                    int col0, int cols_left, int N, float alpha,
                                                    float beta, __amdgpu_buffer_rsrc_t rw,
                                                    int ldw, const float *bias = nullptr,
                                                    int act = kActNone) {
    store_c_bands_lds128<MI, MODE, PLOAD, EPI>(band_writer32<MI>(acc), region, rc, row0, col0,
                                               cols_left, N, alpha, beta, rw, ldw, bias, act);
}

// TRANSB: B is stored N x K (row n holds B[.][n] along k, as attention's
// K): its tile (BN rows n, 64 k) is copied, laid out and read exactly like
// A's.  STAGED (128 x 128 only): the epilogue goes through LDS
// (store_c_tile_lds, whole 256-byte row segments per store) instead of
// 16-byte stores straight from the accumulators.
template <int BM, int BN, bool KTAIL, bool EPI, bool TRANSB = false, bool STAGED = false,
          int S = 2>
__global__ __launch_bounds__(kThreads, 1) void bf16_mfma_kernel(int M, int N, int K, float alpha,
                                                                float beta,
                                                                const uint16_t *__restrict__ A,
                                                                const uint16_t *__restrict__ B,
                                                                float *C, int tiles_m,
                                                                int tiles_n, Epi epi,
                                                                Batch batch) {
    using T = Tile<BM, BN>;
    static_assert(S >= 2, "at least two stages");
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S][T::A_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S][T::B_STAGE];

    // XCD-aware order over the tiles of all items (one item: the plain GEMM)
    int tm, tn;
    const int v = xcd_remap(blockIdx.x, gridDim.x);
    const int per_item = tiles_m * tiles_n;
    const int item = v / per_item;
    A += item * batch.stride_a;
    B += item * batch.stride_b;
    C += item * batch.stride_c;
    grouped_tile(v - item * per_item, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // ---- per-lane global offsets of this wave's direct-to-LDS loads --------
    // A load L = wave + 4 i covers tile rows 8L .. 8L+7; lane p fills chunk
    // position p % 8 of row 8L + p / 8 with logical chunk (p % 8) ^ swz_a(row).
    // The key of that row is the same for every i (8L = 8 wave + 32 i).
    const int a_row_in = lane >> 3;
    const int a_chunk = (lane & 7) ^ swz_a(8 * wave + a_row_in);
    // B load L = wave + 4 i covers rows L * R .. L * R + R - 1 (R rows per KB).
    const int b_row_in = lane / T::B_CHUNKS;
    const int b_pos = lane % T::B_CHUNKS;

    // Wave-load L = wave + 4 i of A covers tile rows 32 i + 8 wave .. +7, of
    // B tile rows 4 R i + R wave .. +R-1 (R rows per 1 KB).  The per-lane
    // offset of load i is the offset of load 0 plus i times a row stride, so
    // one offset register per operand is kept.  Rows past M (A) or K (B) lie
    // beyond the descriptor's range; a column chunk past N is redirected out
    // of range once here, a k chunk past K (only in a K tail) per tile.
    const uint32_t a_off =
        static_cast<uint32_t>(((8 * wave + a_row_in) * K + 8 * a_chunk) * 2);
    const uint32_t a_step = static_cast<uint32_t>(32 * K * 2);
    const int b_row0 = T::B_ROWS_PER_LOAD * wave + b_row_in;  // row of load i = 0
    const int b_c = b_pos ^ swz_b(b_row0);                     // same for every i
    const bool b_ok = (n0 + 8 * b_c) < N;
    const uint32_t b_off = static_cast<uint32_t>((b_row0 * N + 8 * b_c) * 2);
    const uint32_t b_step = static_cast<uint32_t>(4 * T::B_ROWS_PER_LOAD * N * 2);

    // Direct copies of one K tile: loads 0 .. A_LOADS-1 are A, the rest B.
    struct TileCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool a_ok;
    };
    static_assert(!TRANSB || T::B_LOADS == BN / 32, "a transposed B tile copies like A's");
    auto tile_copy = [&](int k0, int stage) {
        TileCopy c;
        // descriptors based at the tile origin
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         (static_cast<long long>(M - m0) * K - k0) * 2);
        if constexpr (TRANSB)
            c.rb = make_desc(B + static_cast<size_t>(n0) * K + k0,
                             (static_cast<long long>(N - n0) * K - k0) * 2);
        else
            c.rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                             (static_cast<long long>(K - k0) * N - n0) * 2);
        c.a_ok = !(KTAIL && k0 + 8 * a_chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 512]);
        c.lb = lds_address(&lds_b[stage][wave * 512]);
        return c;
    };
    auto issue_copy = [&](const TileCopy &c, int q) {
        if (q < T::A_LOADS)
            lds_dma16(c.ra, c.la + q * 4 * 1024, c.a_ok ? a_off + q * a_step : kOOB);
        else if constexpr (TRANSB)
            lds_dma16(c.rb, c.lb + (q - T::A_LOADS) * 4 * 1024,
                      c.a_ok ? a_off + (q - T::A_LOADS) * a_step : kOOB);
        else
            lds_dma16(c.rb, c.lb + (q - T::A_LOADS) * 4 * 1024,
                      b_ok ? b_off + (q - T::A_LOADS) * b_step : kOOB);
    };
    auto issue_tile = [&](int k0, int stage) {
        const TileCopy c = tile_copy(k0, stage);
#pragma unroll
        for (int q = 0; q < T::A_LOADS + T::B_LOADS; ++q) issue_copy(c, q);
    };

    // ---- fragment reads ----------------------------------------------------
    // A: row wm*WM + 32 i + l32, chunk 2 s + h at position chunk ^ swz_a(l32)
    //    (WM and 32 i are multiples of 16, so the key depends on l32 only).
    // B: lane's transposed-read address: row 16 s + 8 h' + 4 r + j / 4 and
    //    columns n_frag + 4 (j % 4), where j = lane % 16, h' = (lane / 32).
    const int a_lane_base = (wm * T::WM + l32) * kBK;
    const int g = lane >> 4, j16 = lane & 15;
    const int b_col_lane = wn * T::WN + 16 * (g & 1) + 4 * (j16 & 3);  // + 32 j
    const int b_row_lane = 8 * (g >> 1) + (j16 >> 2);                  // + 16 s + 4 r

    // Fragment read number q of k16 sub-step s: q < MI reads A block q, the
    // rest read half (q - MI) % 2 of B block (q - MI) / 2 (TRANSB: all of B
    // block q - MI, read like an A block).
    constexpr int kReads = T::MI + (TRANSB ? 1 : 2) * T::NI;
    const int bt_lane_base = (wn * T::WN + l32) * kBK;
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    auto read_one = [&](int stage, int s, int q, bf16x8 (&a)[T::MI], s16x8 (&b)[T::NI]) {
        if (q < T::MI) {
            const int pos = ((2 * s + h) ^ swz_a(l32)) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &lds_a[stage][a_lane_base + 32 * q * kBK + pos]);
            a[q] = __builtin_bit_cast(bf16x8, v);
        } else if constexpr (TRANSB) {
            const int pos = ((2 * s + h) ^ swz_a(l32)) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &lds_b[stage][bt_lane_base + 32 * (q - T::MI) * kBK + pos]);
            b[q - T::MI] = __builtin_bit_cast(s16x8, v);
        } else {
            const int jj = (q - T::MI) >> 1, r = (q - T::MI) & 1;
            const int row = 16 * s + 4 * r + b_row_lane;
            const int col = b_col_lane + 32 * jj;
            const int chunk = (col >> 3) ^ swz_b(row);
            const int elem = row * BN + chunk * 8 + (col & 7);
            const s16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)&lds_b[stage][elem]);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[jj][4 * r + e] = part[e];
        }
    };
    auto read_frags = [&](int stage, int s, bf16x8 (&a)[T::MI], s16x8 (&b)[T::NI]) {
#pragma unroll
        for (int q = 0; q < kReads; ++q) read_one(stage, s, q, a, b);
    };

    f32x16 acc[T::MI][T::NI];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

    const int ktiles = (K + kBK - 1) / kBK;
    constexpr int kCopies = T::A_LOADS + T::B_LOADS;
    // vmcnt <= copies of S - 2 tiles and lgkmcnt == 0
    constexpr int kWaitAhead = ((S - 2) * kCopies & 15) | (7 << 4) | (((S - 2) * kCopies >> 4) << 14);
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
        if (u == 0 || u < ktiles) issue_tile(u * kBK, u);
    if (S == 2 || ktiles < S - 1)
        __builtin_amdgcn_s_waitcnt(0);
    else
        __builtin_amdgcn_s_waitcnt(kWaitAhead);
    __syncthreads();

    // Software pipeline of one K step (tile t in stage t % S):
    //   issue direct loads of tile t+S-1 into the stage tile t-1 used
    //   sub-steps 0..2: read fragments of sub-step s+1, 16 MFMAs of sub-step s
    //   sub-step 3:     wait for own loads of tile t+1 + barrier (the
    //                   current stage is then no longer read and tile t+1 is
    //                   complete), read tile t+1's sub-step-0 fragments, 16
    //                   MFMAs of sub-step 3
    // With two stages, past the last tile the "next" tile lies beyond K, so
    // its loads are all out of range and only write zeros into the idle
    // stage; with more, tiles past K are not copied, and the last S - 1
    // steps wait for every copy.  Scheduling barriers keep each sub-step's
    // fragment reads (and the step's global loads) interleaved with its
    // MFMAs.
    bf16x8 fa[2][T::MI];
    s16x8 fb[2][T::NI];
    read_frags(0, 0, fa[0], fb[0]);
    constexpr int kMfma = T::MI * T::NI;
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t % S;
        const bool ahead = t + S - 1 < ktiles;  // tile t + S - 1 exists
        const TileCopy copy = tile_copy((t + S - 1) * kBK, (t + S - 1) % S);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int f = s & 1;
            const bool last = (s + 1 == kBK / 16);
            // Manual schedule: MFMA q is followed by fragment read q of the
            // next sub-step and, in sub-step 0, by global->LDS copy q.  In
            // the last sub-step the first half of the MFMAs runs before the
            // barrier and the next tile's reads follow it.
            constexpr int kHalf = kMfma / 2;
            constexpr int kReadsPerSlot = (kReads + kMfma - 1) / kMfma;
            constexpr int kReadsPerLateSlot = (kReads + (kMfma - kHalf) - 1) / (kMfma - kHalf);
            constexpr int kCopiesPerSlot = (kCopies + kMfma - 1) / kMfma;
#pragma unroll
            for (int q = 0; q < kMfma; ++q) {
                const int i = q / T::NI, jj = q % T::NI;
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, fb[f][jj]), fa[f][i], acc[i][jj], 0, 0, 0);
                if (!last) {
#pragma unroll
                    for (int u = 0; u < kReadsPerSlot; ++u) {
                        const int rq = q * kReadsPerSlot + u;
                        if (rq < kReads) read_one(cur, s + 1, rq, fa[f ^ 1], fb[f ^ 1]);
                    }
                    if (s == 0 && (S == 2 || ahead)) {
#pragma unroll
                        for (int u = 0; u < kCopiesPerSlot; ++u) {
                            const int cq = q * kCopiesPerSlot + u;
                            if (cq < kCopies) issue_copy(copy, cq);
                        }
                    }
                } else {
                    if (q == kHalf - 1) {
                        // own copies of tile t+1 landed ...
                        if (S == 2 || !ahead)
                            __builtin_amdgcn_s_waitcnt(0);
                        else
                            __builtin_amdgcn_s_waitcnt(kWaitAhead);
                        __syncthreads();  // ... and everyone else's
                    }
                    if (q >= kHalf) {
#pragma unroll
                        for (int u = 0; u < kReadsPerLateSlot; ++u) {
                            const int rq = (q - kHalf) * kReadsPerLateSlot + u;
                            if (rq < kReads)
                                read_one((t + 1) % S, 0, rq, fa[f ^ 1], fb[f ^ 1]);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- epilogue
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    if constexpr (STAGED) {
        // every wave's last reads are done before any wave reuses a stage
        // (and, the last step having waited for every copy, no copy is in
        // flight): waves 0 and 1 stage through A stages 0 and 1, 2 and 3
        // through B stages 0 and 1
        static_assert(T::NI == 2 && T::A_STAGE * 2 >= 16384 && T::B_STAGE * 2 >= 16384,
                      "64-column wave tiles, 16 KB stages");
        __syncthreads();
        float *region = reinterpret_cast<float *>(wave < 2 ? &lds_a[wave][0] : &lds_b[wave - 2][0]);
        store_c_tile_lds<T::MI, T::NI, kStoreC, kSystemScope, EPI>(
            acc, region, rc, wm * T::WM, wn * T::WN, N - n0, N, alpha, beta, rc, 0,
            EPI && epi.bias ? epi.bias + n0 : nullptr, epi.act);
    } else {
        store_c_tile<T::MI, T::NI, EPI>(acc, rc, wm * T::WM, wn * T::WN, N - n0, N, alpha, beta,
                                        epi.bias ? epi.bias + n0 : nullptr, epi.act);
    }
}

// ---------------------------------------------------------------------------
// Ping-pong variant: 512 threads = 8 waves, two per SIMD, K step 32 and S
// LDS stages.  The waves form two groups of four (group = wave / 4, one wave
// of each group per SIMD) that alternate between a read phase (all MFMA
// fragments of one K step from LDS into registers) and a compute phase (all
// MFMAs of that K step), group 1 one phase behind group 0, with a workgroup
// barrier between phases.  While one wave of a SIMD runs back-to-back MFMAs
// the other issues its LDS reads, so the matrix core is not stalled by the
// reads of the wave that feeds it (the single-wave kernel above pays for
// every read slotted between its MFMAs).
//
// Global -> LDS copies run S - 1 K steps ahead.  The stage of step t+S-1 is
// the stage of step t-1, free once both groups have read step t-1, i.e.
// after barrier B_{2t}.  Both groups copy during their compute phases, one
// copy after every few MFMAs (a compute phase then has no branches, and the
// per-CU copy rate stays well below the L2 -> LDS limit of about 64 bytes
// per clock): group 1 copies its share of step t+S-1 in its compute phase
// of step t-1 (after B_{2t}), group 0 its share in its compute phase of step
// t (after B_{2t+1}).  Each wave waits for its own copies of step t+1 before
// the barrier after which step t+1 is first read (group 0 at the end of its
// compute phase of step t, group 1 at the end of its read phase of step t):
// copies have at least 2 S - 3 phases to land.
//
// LDS layouts (64-bank LDS, see the notes at the top): A stage = BM rows of
// 32 k (64 bytes, 4 chunks), chunk c of row r at position c ^ ((r / 4) % 4),
// so that 16 consecutive rows of one chunk cover the 64 banks; B stage = 32
// k-rows of BN n, swizzled with swz_b as above.
//
// Barrier schedule (B_n = n-th barrier, T = number of K steps):
//   all:     copy steps 0 .. S-2, wait for step 0, B_0
//   group 1: copy its share of step S-1, B_1
//   group 0: read(t) B_{2t+1} compute(t) B_{2t+2}            t = 0 .. T-1
//   group 1: read(t) B_{2t+2} compute(t) B_{2t+3}            (no B after
//            compute(T-1): both groups execute exactly 2T + 1 barriers)
// so group 0 computes step t while group 1 reads it, and group 0 reads step
// t+1 while group 1 computes step t.  Group 0's epilogue overlaps group 1's
// last compute phase.
constexpr int kPPBK = 32;

template <int BM, int BN>
struct PPTile {
    static constexpr int WAVES_M = (BN == 256) ? 2 : 4;
    static constexpr int WAVES_N = 8 / WAVES_M;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // wave tile
    static constexpr int MI = WM / 32, NI = WN / 32;
    static constexpr int A_LOADS = BM / 16 / 8;      // 1 KB copies of A per wave per step
    static constexpr int B_ROWS = 512 / BN;          // B rows per 1 KB copy
    static constexpr int B_LOADS = kPPBK / B_ROWS / 8;  // 1 KB copies of B per wave per step
    static constexpr int COPIES = A_LOADS + B_LOADS;
    static constexpr int B_CHUNKS = BN / 8;          // 16-byte chunks per B row
    static constexpr int A_STAGE = BM * kPPBK;       // bf16 elements
    static constexpr int B_STAGE = kPPBK * BN;
};

__device__ __forceinline__ int swz_a32(int r) { return (r >> 2) & 3; }


// ---- the split pair's handshake (see PPSplit) ------------------------------
// LOCAL pairs share one XCD and exchange through ordinary memory whose
// coherence point for both is that XCD's L2: device (agent) scope.  Other
// pairs exchange through uncached memory: system scope.  Each function is
// called by every thread of the workgroup; `word` is an LDS int used to
// broadcast thread 0's result, a different one for each function.

// The split index of this workgroup: 0 if it is the first of its pair to
// claim the tile, 1 if the second.  Called at the kernel's start: thread 0
// swaps the epoch into the tile's claim word (the swap only decides the
// roles, so it needs no ordering of its own).  The first to claim is then
// running and never waits, so the second, which waits for it, waits for a
// workgroup that will finish.
template <bool LOCAL>
__device__ __forceinline__ int pair_arrive(const PPSplit &p, int slot, int *word) {
    if (threadIdx.x == 0) {
        const unsigned old =
            LOCAL ? __hip_atomic_exchange(p.claims + slot, p.epoch, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                  : __hip_atomic_exchange(p.claims + slot, p.epoch, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
        *word = old == p.epoch;
    }
    __syncthreads();
    return *word;
}

// The first of a pair, after every wave has stored its share of the partial
// tile: the barrier orders all of them before thread 0's release store of
// the flag.
template <bool LOCAL>
__device__ __forceinline__ void pair_publish(const PPSplit &p, int slot) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        if (LOCAL)
            __hip_atomic_store(p.flags + slot, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(p.flags + slot, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// The second of a pair: wait until the first has published its partial.
// Thread 0 polls with relaxed loads, at most poll_limit of them, and then
// takes an acquire fence; the barrier hands the ordering on to the other
// waves.  Returns false (after counting the time-out) if the flag never
// came; the first workgroup of the pair is already past its K loop, so that
// only happens when poll_limit is too small for the partial's store.
template <bool LOCAL>
__device__ __forceinline__ bool pair_wait(const PPSplit &p, int slot, int *word) {
    if (threadIdx.x == 0) {
        int ready = 0;
        for (int poll = 0; poll < p.poll_limit; ++poll) {
            const unsigned f =
                LOCAL ? __hip_atomic_load(p.flags + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : __hip_atomic_load(p.flags + slot, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_SYSTEM);
            if (f == p.epoch) {
                ready = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (ready) {
            if (LOCAL)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            else
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
        } else if (p.timeouts != nullptr) {
            __hip_atomic_fetch_add(p.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        *word = ready;
    }
    __syncthreads();
    return *word != 0;
}

// Tile and K half of workgroup `bid` under a split plan: workgroups below
// split_from own a whole tile (XCD-aware order, split = -1); the rest come
// in pairs that share a tile.  With xcd_pairs, workgroups b and b + 8 pair
// up (one XCD under round-robin dealing), else 2i and 2i + 1.  Of a pair,
// the first to claim the tile (pair_arrive) is split 0, which takes the K
// steps before split_step and posts its partial; the other is split 1,
// which takes the rest, waits for the partial and writes C.  So the
// workgroup that started first gets the shorter half, and the one that
// waits only ever waits for a running workgroup.  Every thread of the
// workgroup calls this (it has a barrier when the tile is split).
__device__ __forceinline__ void split_tile(int bid, const PPSplit &plan, int &v, int &split,
                                           int *word) {
    split = -1;
    if (bid < plan.split_from) {
        v = xcd_remap(bid, plan.split_from);
        return;
    }
    const int q = bid - plan.split_from;
    if (plan.xcd_pairs) {
        const int p = (q >> 4) * 8 + (q & 7);
        v = plan.split_from + xcd_remap(p, plan.grid_tiles - plan.split_from);
        split = pair_arrive<true>(plan, v - plan.split_from, word);
    } else {
        v = plan.split_from + (q >> 1);
        split = pair_arrive<false>(plan, v - plan.split_from, word);
    }
}

template <int BM, int BN, int S, bool KTAIL, bool EPI>
__global__ __launch_bounds__(512, 1) void bf16_pp_kernel(int M, int N, int K, float alpha,
                                                         float beta,
                                                         const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B, float *C,
                                                         int tiles_m, int tiles_n,
                                                         PPSplit split_plan, Epi epi) {
    using T = PPTile<BM, BN>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S][T::A_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S][T::B_STAGE];

    // Tile and K range of this workgroup.  Workgroups below split_from own a
    // whole tile (XCD-aware order); the rest come in pairs that share one of
    // the remaining tiles: the first takes the K steps below split_step and
    // posts its partial sums, the second takes the rest and adds them.
    int v, split;
    __shared__ int s_role, s_ready;
    split_tile(blockIdx.x, split_plan, v, split, &s_role);
    int tm, tn;
    grouped_tile(v, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int total_steps = (K + kPPBK - 1) / kPPBK;
    const int t_begin = split == 1 ? split_plan.split_step : 0;
    const int t_end = split == 0 ? split_plan.split_step : total_steps;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const int l32 = lane & 31, h = lane >> 5;

    // ---- this wave's copies.  A copy q is wave-load L = 8 q + wave: tile
    // rows 16 L .. 16 L + 15, lane p filling position p % 4 of row
    // 16 L + p / 4 with logical chunk (p % 4) ^ swz_a32(row) (the key is
    // (p / 16) % 4 for every L).  B copy q is wave-load 8 q + wave: B_ROWS
    // rows from row B_ROWS (8 q + wave); the key of a row does not depend
    // on q.
    const int a_row_in = lane >> 2;
    const int a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t a_off =
        static_cast<uint32_t>(((16 * wave + a_row_in) * K + 8 * a_chunk) * 2);
    const uint32_t a_step = static_cast<uint32_t>(128 * K * 2);
    const int b_row0 = T::B_ROWS * wave + lane / T::B_CHUNKS;
    const int b_c = (lane % T::B_CHUNKS) ^ swz_b(b_row0);
    const bool b_ok = (n0 + 8 * b_c) < N;
    const uint32_t b_off = static_cast<uint32_t>((b_row0 * N + 8 * b_c) * 2);
    const uint32_t b_step = static_cast<uint32_t>(8 * T::B_ROWS * N * 2);

    struct StepCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool a_ok;
    };
    auto step_copy = [&](int t) {
        const int k0 = (t_begin + t) * kPPBK, stage = t % S;
        StepCopy c;
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         (static_cast<long long>(M - m0) * K - k0) * 2);
        c.rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                         (static_cast<long long>(K - k0) * N - n0) * 2);
        c.a_ok = !(KTAIL && k0 + 8 * a_chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 512]);
        c.lb = lds_address(&lds_b[stage][wave * 512]);
        return c;
    };
    auto issue_copy = [&](const StepCopy &c, int q) {
        if (q < T::A_LOADS)
            lds_dma16(c.ra, c.la + q * 8 * 1024, c.a_ok ? a_off + q * a_step : kOOB);
        else
            lds_dma16(c.rb, c.lb + (q - T::A_LOADS) * 8 * 1024,
                      b_ok ? b_off + (q - T::A_LOADS) * b_step : kOOB);
    };
    auto issue_step = [&](int t) {
        const StepCopy c = step_copy(t);
#pragma unroll
        for (int q = 0; q < T::COPIES; ++q) issue_copy(c, q);
    };

    // ---- fragments of one K step: A block i, k16 step s; B block jj, step s
    const int a_lane_base = (wm * T::WM + l32) * kPPBK;
    const int g = lane >> 4, j16 = lane & 15;
    const int b_col_lane = wn * T::WN + 16 * (g & 1) + 4 * (j16 & 3);  // + 32 jj
    const int b_row_lane = 8 * (g >> 1) + (j16 >> 2);                  // + 16 s + 4 r
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    constexpr int kSub = kPPBK / 16;
    constexpr int kReads = kSub * (T::MI + 2 * T::NI);
    bf16x8 fa[T::MI][kSub];
    s16x8 fb[T::NI][kSub];
    s16x4 fb_part[T::NI][kSub][2];
    // Fragment read number q of the step (A blocks first, then B halves).
    auto read_one = [&](int stage, int q) {
        constexpr int per_s = T::MI + 2 * T::NI;
        const int s = q / per_s, u = q % per_s;
        if (u < T::MI) {
            const int pos = ((2 * s + h) ^ swz_a32(l32)) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &lds_a[stage][a_lane_base + 32 * u * kPPBK + pos]);
            fa[u][s] = __builtin_bit_cast(bf16x8, v);
        } else {
            const int jj = (u - T::MI) >> 1, r = (u - T::MI) & 1;
            const int row = 16 * s + 4 * r + b_row_lane;
            const int col = b_col_lane + 32 * jj;
            const int chunk = (col >> 3) ^ swz_b(row);
            const int elem = row * BN + chunk * 8 + (col & 7);
            fb_part[jj][s][r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)&lds_b[stage][elem]);
        }
    };

    f32x16 acc[T::MI][T::NI];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

    const int steps = t_end - t_begin;
    constexpr int kWaitSteady = wait_vm(T::COPIES * (S - 2));
    constexpr int kWaitAll = wait_vm(0);
    for (int t = 0; t < S - 1; ++t)
        if (t < steps) issue_step(t);
    if (steps >= S - 1)
        __builtin_amdgcn_s_waitcnt(kWaitSteady);  // step 0 landed
    else
        __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();  // B_0
    if (grp == 1) {
        if (S - 1 < steps) issue_step(S - 1);
        __syncthreads();  // B_1
    }

    constexpr int kMfma = T::MI * T::NI * kSub;
    constexpr int kGapM = kMfma / T::COPIES;
    // One K step: read phase, barrier, compute phase, barrier.  With COPY the
    // compute phase also copies step t + S - 1 + grp (one copy after every
    // kGapM-th MFMA) and the waits keep the younger steps in flight; without
    // it (the last steps) every wait drains the queue.
    auto k_step = [&](int t, auto copy_tag) {
        constexpr bool COPY = decltype(copy_tag)::value;
        const int stage = t % S;
#pragma unroll
        for (int q = 0; q < kReads; ++q) read_one(stage, q);
        if (grp == 1) __builtin_amdgcn_s_waitcnt(COPY ? kWaitSteady : kWaitAll);
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj)
#pragma unroll
            for (int s = 0; s < kSub; ++s)
                fb[jj][s] = __builtin_shufflevector(fb_part[jj][s][0], fb_part[jj][s][1], 0, 1, 2,
                                                    3, 4, 5, 6, 7);
        StepCopy next;
        if (COPY) next = step_copy(t + S - 1 + grp);
#pragma unroll
        for (int q = 0; q < kMfma; ++q) {
            const int s = q / (T::MI * T::NI);
            const int i = (q / T::NI) % T::MI, jj = q % T::NI;
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fb[jj][s]), fa[i][s], acc[i][jj], 0, 0, 0);
            if (COPY && q % kGapM == 0 && q / kGapM < T::COPIES) issue_copy(next, q / kGapM);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (grp == 0) {
            __builtin_amdgcn_s_waitcnt(COPY ? kWaitSteady : kWaitAll);
            __syncthreads();
        } else if (t + 1 < steps) {
            __syncthreads();
        }
    };
    // Steps whose compute phase copies: group 0 copies step t + S - 1, group
    // 1 step t + S, while that step exists.
    const int copy_end = max(0, steps - (S - 1) - grp);
    int t = 0;
    for (; t < copy_end; ++t) k_step(t, std::true_type());
    for (; t < steps; ++t) k_step(t, std::false_type());

    // ---- epilogue
    // ---- epilogue.  After the last barrier no wave reads the LDS stages and
    // no copy is in flight (every wave drained its copies before it), so
    // each wave stages its tile through a private 16 KB slice of them:
    // waves 0-3 (which finish first) in the A stages, waves 4-7 in the B
    // stages.
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    static_assert(T::WN == 64 && S * T::A_STAGE * 2 >= 4 * 16384 &&
                      S * T::B_STAGE * 2 >= 4 * 16384,
                  "the epilogue stages 16 KB per wave through the LDS stages");
    float *region = wave < 4 ? reinterpret_cast<float *>(&lds_a[0][0]) + wave * 4096
                             : reinterpret_cast<float *>(&lds_b[0][0]) + (wave - 4) * 4096;
    const int row0 = wm * T::WM, col0 = wn * T::WN;
    const float *bias = EPI && epi.bias ? epi.bias + n0 : nullptr;  // tile's first column
    if (split < 0) {
        store_c_tile_lds<T::MI, T::NI, kStoreC, kSystemScope, EPI>(
            acc, region, rc, row0, col0, N - n0, N, alpha, beta, rc, 0, bias, epi.act);
        return;
    }
    // A split tile: its partial lives in the workspace slot of the pair.
    const int slot = v - split_plan.split_from;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(split_plan.partials + static_cast<size_t>(slot) * BM * BN, BM * BN * 4);
    const bool local = split_plan.xcd_pairs != 0;
    if (split == 0) {
        store_c_tile_lds<T::MI, T::NI, kPostPartial>(acc, region, rc, row0, col0, N - n0, N,
                                                     alpha, beta, rw, BN);
        if (local)
            pair_publish<true>(split_plan, slot);
        else
            pair_publish<false>(split_plan, slot);
        return;
    }
    const bool ok = local ? pair_wait<true>(split_plan, slot, &s_ready)
                          : pair_wait<false>(split_plan, slot, &s_ready);
    const float a = ok ? alpha : __builtin_nanf("");
    // partial loads: device scope (skip the CU's L1) for pairs on one XCD,
    // system scope through uncached memory otherwise
    if (local)
        store_c_tile_lds<T::MI, T::NI, kAddPartial, kDeviceScope, EPI>(
            acc, region, rc, row0, col0, N - n0, N, a, beta, rw, BN, bias, epi.act);
    else
        store_c_tile_lds<T::MI, T::NI, kAddPartial, kSystemScope, EPI>(
            acc, region, rc, row0, col0, N - n0, N, a, beta, rw, BN, bias, epi.act);
}


// The epilogue of a 256 x 256 four-wave tile under a split plan: a whole
// tile stores alpha acc + beta C; of a split pair, split 0 posts its partial
// to the pair's workspace slot and publishes it, split 1 waits for it
// (pair_wait: on time-out it writes NaN rather than hang) and stores alpha
// (acc + partial) + beta C.  `word` is an LDS int the workgroup no longer
// uses (it broadcasts the wait's outcome).  The wave's accumulators reach
// the epilogue through write_band (see store_c_bands_lds128).
template <int BANDS, bool EPI, class WriteBand>
__device__ __forceinline__ void store_split_bands(WriteBand &&wb, float *region,
                                                  __amdgpu_buffer_rsrc_t rc, int row0, int col0,
                                                  int cols_left, int N, float alpha, float beta,
                                                  int split, int v, const PPSplit &split_plan,
                                                  const float *bias, int act, int *word) {
    constexpr int BN = kPPTile;
    if (split < 0) {
        store_c_bands_lds128<BANDS, kStoreC, kSystemScope, EPI>(wb, region, rc, row0, col0,
                                                                cols_left, N, alpha, beta, rc, 0,
                                                                bias, act);
        return;
    }
    const int slot = v - split_plan.split_from;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(split_plan.partials + static_cast<size_t>(slot) * BN * BN, BN * BN * 4);
    const bool local = split_plan.xcd_pairs != 0;
    if (split == 0) {
        store_c_bands_lds128<BANDS, kPostPartial>(wb, region, rc, row0, col0, cols_left, N,
                                                  alpha, beta, rw, BN);
        if (local)
            pair_publish<true>(split_plan, slot);
        else
            pair_publish<false>(split_plan, slot);
        return;
    }
    const bool ok = local ? pair_wait<true>(split_plan, slot, word)
                          : pair_wait<false>(split_plan, slot, word);
    const float a = ok ? alpha : __builtin_nanf("");
    if (local)
        store_c_bands_lds128<BANDS, kAddPartial, kDeviceScope, EPI>(
            wb, region, rc, row0, col0, cols_left, N, a, beta, rw, BN, bias, act);
    else
        store_c_bands_lds128<BANDS, kAddPartial, kSystemScope, EPI>(
            wb, region, rc, row0, col0, cols_left, N, a, beta, rw, BN, bias, act);
}

template <int MI, bool EPI>
__device__ __forceinline__ void store_split_tile(const f32x16 (&acc)[MI][4], float *region,
                                                 __amdgpu_buffer_rsrc_t rc, int row0, int col0,
                                                 int cols_left, int N, float alpha, float beta,
                                                 int split, int v, const PPSplit &split_plan,
                                                 const float *bias, int act, int *word) {
    store_split_bands<MI, EPI>(band_writer32<MI>(acc), region, rc, row0, col0, cols_left, N, alpha,
                               beta, split, v, split_plan, bias, act, word);
}

// ---------------------------------------------------------------------------
// Four-wave 256 x 256 kernel on the ping-pong kernel's 32-k LDS layout:
// 256 threads = four waves in 2 x 2, each owning a 128 x 128 wave tile (256
// fp32 accumulators per lane, the whole AccVGPR file), K step 32, four LDS
// stages (128 KB) filled by direct global -> LDS copies three K steps ahead.
// Against the ping-pong kernel it reads a third less LDS per MFMA (128 x 128
// wave tiles instead of 128 x 64), but a single wave per SIMD must hide its
// own LDS reads and copies:
//   * one K step = the last 8 MFMAs of the previous step's second k16
//     sub-step (with this step's first fragment reads), the 16 MFMAs of
//     sub-step 0 (with the reads of sub-step 1), the first 8 MFMAs of
//     sub-step 1, a wait and a barrier.  An iteration ends at the barrier,
//     where no LDS read is outstanding, so the compiler's wait counts inside
//     the body are exact; reads are issued in the order the MFMAs use them
//     (consecutive MFMAs share a B fragment);
//   * the eight 1 KB copies of step t + 3 are spread over the step, one per
//     four MFMAs in sub-step 0 and one per two after it.  Issuing them in a
//     burst stalled the MFMA stream behind the copy queue (timing-only copies
//     of the kernel: with L2-resident copies and no fragment reads it still
//     took 40 % longer than with no copies at all);
//   * the wait before the barrier leaves the copies of steps t + 2 and t + 3
//     in flight and requires those of step t + 1 and every fragment read:
//     the next stage is complete for every wave and the stage that step t +
//     4's copies will overwrite is no longer read.
// Edges: rows past M and B rows past K lie outside the copy descriptors
// (zero-filled), columns past N are redirected out of range, A chunks past K
// (a K tail) are skipped per step.  The epilogue stages each wave's tile
// through LDS (store_c_tile_lds128), about 1 % faster than direct 16-byte
// stores.
template <bool KTAIL, bool EPI, bool TRANSB, bool PERSIST = false>
__global__ __launch_bounds__(256, 1) void bf16_q4_kernel(int M, int N, int K, float alpha,
                                                         float beta,
                                                         const uint16_t *__restrict__ A0,
                                                         const uint16_t *__restrict__ B0, float *C0,
                                                         int tiles_m, int tiles_n,
                                                         PPSplit split_plan, Epi epi,
                                                         Batch batch) {
    constexpr int BM = 256, BN = 256, S = 4, BK = kPPBK;
    constexpr int WM = 128, WN = 128, MI = 4, NI = 4;
    constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;
    constexpr int A_LOADS = BM / 16 / 4;
    constexpr int B_ROWS = 512 / BN;
    constexpr int B_LOADS = BK / B_ROWS / 4;
    constexpr int COPIES = A_LOADS + B_LOADS;
    constexpr int B_CHUNKS = BN / 8;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S][A_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S][B_STAGE];

    // Tile and K range: as in the ping-pong kernel, workgroups below
    // split_from own a whole tile (XCD-aware order) and the rest come in
    // pairs that share a tile, one per half of the K steps.  PERSIST (a
    // batched launch, never split, on a grid that is a multiple of 8 and
    // smaller than the tile count): workgroup b takes the tiles that
    // workgroups b, b + grid, b + 2 grid, ... would take, all on its XCD.
    int v, split;
    __shared__ int s_words[2];
    const int per_item = tiles_m * tiles_n;
    const uint16_t *A, *B;
    float *C;
    int m0, n0;
    // A batched launch (never split) numbers the tiles of all items in
    // turn: the XCD-aware order keeps one item's tiles on one XCD.
    auto set_tile = [&](int bid) {
        if constexpr (PERSIST) {
            v = xcd_remap(bid, split_plan.grid_tiles);
            split = -1;
        } else {
            split_tile(bid, split_plan, v, split, &s_words[0]);
        }
        const int item = v / per_item;
        A = A0 + item * batch.stride_a;
        B = B0 + item * batch.stride_b;
        C = C0 + item * batch.stride_c;
        int tm, tn;
        grouped_tile(v - item * per_item, tiles_m, tiles_n, 4, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
    };
    int bid = blockIdx.x;
    set_tile(bid);
    const int total_steps = (K + BK - 1) / BK;
    const int t_begin = split == 1 ? split_plan.split_step : 0;
    const int t_end = split == 0 ? split_plan.split_step : total_steps;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    const int a_row_in = lane >> 2;
    const int a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t a_off = static_cast<uint32_t>(((16 * wave + a_row_in) * K + 8 * a_chunk) * 2);
    const uint32_t a_step = static_cast<uint32_t>(64 * K * 2);
    const int b_row0 = B_ROWS * wave + lane / B_CHUNKS;
    const int b_c = (lane % B_CHUNKS) ^ swz_b(b_row0);
    bool b_ok = (n0 + 8 * b_c) < N;
    const uint32_t b_off = static_cast<uint32_t>((b_row0 * N + 8 * b_c) * 2);
    const uint32_t b_step = static_cast<uint32_t>(4 * B_ROWS * N * 2);

    struct StepCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool a_ok;
    };
    // TRANSB: B is stored N x K (row n holds B[.][n] along k), so its tile
    // (256 rows n, 32 k) is copied and laid out exactly like A's tile.
    static_assert(!TRANSB || B_LOADS == A_LOADS, "a transposed B tile copies like A's");
    auto step_copy = [&](int t) {  // t counts this workgroup's steps
        const int k0 = (t_begin + t) * BK, stage = t % S;
        StepCopy c;
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         (static_cast<long long>(M - m0) * K - k0) * 2);
        if constexpr (TRANSB)
            c.rb = make_desc(B + static_cast<size_t>(n0) * K + k0,
                             (static_cast<long long>(N - n0) * K - k0) * 2);
        else
            c.rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                             (static_cast<long long>(K - k0) * N - n0) * 2);
        c.a_ok = !(KTAIL && k0 + 8 * a_chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 512]);
        c.lb = lds_address(&lds_b[stage][wave * 512]);
        return c;
    };
    auto issue_copy = [&](const StepCopy &c, int q) {
        if (q < A_LOADS)
            lds_dma16(c.ra, c.la + q * 4 * 1024, c.a_ok ? a_off + q * a_step : kOOB);
        else if constexpr (TRANSB)
            lds_dma16(c.rb, c.lb + (q - A_LOADS) * 4 * 1024,
                      c.a_ok ? a_off + (q - A_LOADS) * a_step : kOOB);
        else
            lds_dma16(c.rb, c.lb + (q - A_LOADS) * 4 * 1024,
                      b_ok ? b_off + (q - A_LOADS) * b_step : kOOB);
    };

    const int a_lane_base = (wm * WM + l32) * BK;
    const int g = lane >> 4, j16 = lane & 15;
    const int b_col_lane = wn * WN + 16 * (g & 1) + 4 * (j16 & 3);
    const int b_row_lane = 8 * (g >> 1) + (j16 >> 2);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    // fragment reads per sub-step: one per A block, and per B block two
    // transposing reads (B as K x N) or one plain read (TRANSB)
    constexpr int kBReads = TRANSB ? 1 : 2;
    constexpr int kReads = MI + kBReads * NI;
    const int b_lane_base = (wn * WN + l32) * BK;  // TRANSB: row n of the B tile
    auto read_one = [&](int stage, int s, int q, bf16x8 (&a)[MI], s16x8 (&b)[NI]) {
        if (q < MI) {
            const int pos = ((2 * s + h) ^ swz_a32(l32)) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &lds_a[stage][a_lane_base + 32 * q * BK + pos]);
            a[q] = __builtin_bit_cast(bf16x8, v);
        } else if constexpr (TRANSB) {
            const int jj = q - MI;
            const int pos = ((2 * s + h) ^ swz_a32(l32)) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &lds_b[stage][b_lane_base + 32 * jj * BK + pos]);
            b[jj] = __builtin_bit_cast(s16x8, v);
        } else {
            const int jj = (q - MI) >> 1, r = (q - MI) & 1;
            const int row = 16 * s + 4 * r + b_row_lane;
            const int col = b_col_lane + 32 * jj;
            const int chunk = (col >> 3) ^ swz_b(row);
            const int elem = row * BN + chunk * 8 + (col & 7);
            const s16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)&lds_b[stage][elem]);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[jj][4 * r + e] = part[e];
        }
    };
    // reads in consumption order: B block 0, every A block, then the other
    // B blocks
    auto read_in_order = [&](int stage, int s, int r, bf16x8 (&a)[MI], s16x8 (&b)[NI]) {
        const int q = r < kBReads ? MI + r : (r < kBReads + MI ? r - kBReads : r);
        read_one(stage, s, q, a, b);
    };

    f32x16 acc[MI][NI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
    };
    if constexpr (!PERSIST) zero_acc();
    bf16x8 fa[2][MI];
    s16x8 fb[2][NI];
    // MFMA q of a sub-step is block (q % MI, q / MI): consecutive MFMAs
    // share their B fragment (measured 0.5 % faster than sharing A)
    auto mfma = [&](int q, int f) {
        const int jj = q / MI, i = q % MI;
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, fb[f][jj]), fa[f][i], acc[i][jj], 0, 0, 0);
    };
    constexpr int kMfma = MI * NI;
    constexpr int kEarly = 2 * MI;
    constexpr int kTail = kMfma - kEarly;
    // vmcnt <= vm and lgkmcnt == 0
    constexpr int kWaitSteady = (2 * COPIES & 15) | (7 << 4) | ((2 * COPIES >> 4) << 14);
    constexpr int kWaitDrain = (7 << 4);

    const int T = t_end - t_begin;
    auto issue_step = [&](int t) {
        const StepCopy c = step_copy(t);
#pragma unroll
        for (int q = 0; q < COPIES; ++q) issue_copy(c, q);
    };
    for (int t = 0; t < S - 1; ++t)
        if (t < T) issue_step(t);
    if (T >= S - 1)
        __builtin_amdgcn_s_waitcnt(kWaitSteady);
    else
        __builtin_amdgcn_s_waitcnt(kWaitDrain);
    __syncthreads();

    // One K step (stage t % 4): the tail of the previous step's second k16
    // sub-step with this step's first reads; sub-step 0 with the reads of
    // sub-step 1 and the copies of step t + 3; the first MFMAs of sub-step
    // 1; wait for this wave's copies of step t + 1 (and all its reads);
    // barrier.
    auto k_step = [&](int t, auto copy_tag) {
        constexpr bool COPY = decltype(copy_tag)::value;
        const int cur = t % S;
        if (t > 0) {
#pragma unroll
            for (int q = 0; q < kTail; ++q) {
                mfma(kEarly + q, 1);
                constexpr int per = (kReads + kTail - 1) / kTail;
#pragma unroll
                for (int u = 0; u < per; ++u)
                    if (q * per + u < kReads) read_in_order(cur, 0, q * per + u, fa[0], fb[0]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        StepCopy next;
        if (COPY) next = step_copy(t + S - 1);
#pragma unroll
        for (int q = 0; q < kMfma; ++q) {
            mfma(q, 0);
            if (q < kReads) read_in_order(cur, 1, q, fa[1], fb[1]);
            if (COPY && (q & 3) == 0) issue_copy(next, q / 4);  // copies 0..3
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < kEarly; ++q) {
            mfma(q, 1);
            if (COPY && (q & 1) == 0) issue_copy(next, 4 + q / 2);  // copies 4..7
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(COPY ? kWaitSteady : kWaitDrain);
        __syncthreads();
    };
    const int copy_end = max(0, T - (S - 1));
    static_assert(S == 4, "the persistent epilogue takes stage 3 and two more slices");
    const int total_tiles = split_plan.grid_tiles;
    for (;;) {
        if constexpr (PERSIST) zero_acc();
#pragma unroll
        for (int r = 0; r < kReads; ++r) read_in_order(0, 0, r, fa[0], fb[0]);
        int t = 0;
        for (; t < copy_end; ++t) k_step(t, std::true_type());
        for (; t < T; ++t) k_step(t, std::false_type());
#pragma unroll
        for (int q = 0; q < kTail; ++q) {
            mfma(kEarly + q, 1);
            __builtin_amdgcn_sched_barrier(0);
        }

        // After the last barrier no LDS stage is read and no copy is in
        // flight.  Each wave stages its tile through a private 16 KB LDS
        // slice: one of the A stages or, with PERSIST, stage 3's A or B
        // half or one of two more slices (which fill the CU's 160 KB),
        // while the next tile's first three steps are copied into stages 0
        // to 2.
        const __amdgpu_buffer_rsrc_t rc =
            make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                      (static_cast<long long>(M - m0) * N - n0) * 4);
        static_assert(S * A_STAGE * 2 >= 4 * 16384,
                      "four 16 KB epilogue slices fit in the A stages");
        static_assert(A_STAGE * 2 == 16384 && B_STAGE * 2 == 16384, "16 KB stages");
        float *region;
        if constexpr (PERSIST) {
            __shared__ __attribute__((aligned(16))) float lds_x[2][4096];
            region = wave == 0   ? reinterpret_cast<float *>(&lds_a[S - 1][0])
                     : wave == 1 ? reinterpret_cast<float *>(&lds_b[S - 1][0])
                                 : &lds_x[wave - 2][0];
        } else {
            region = reinterpret_cast<float *>(&lds_a[0][0]) + wave * 4096;
        }
        const int row0 = wm * WM, col0 = wn * WN;
        const int tile_n0 = n0, tile_v = v, tile_split = split;
        const float *bias = EPI && epi.bias ? epi.bias + n0 : nullptr;  // tile's first column
        bool more = false;
        if constexpr (PERSIST) {
            bid += gridDim.x;
            more = bid < total_tiles;
            if (more) {
                set_tile(bid);
                b_ok = (n0 + 8 * b_c) < N;
                for (int tt = 0; tt < S - 1; ++tt)
                    if (tt < T) issue_step(tt);
            }
        }
        if constexpr (PERSIST) {
            // The epilogue's row offsets are the same for every tile: an
            // opaque copy of N keeps the compiler from computing them once
            // before the tile loop and holding them (spilled) through it.
            int n_ld = N;
            asm volatile("" : "+s"(n_ld));
            store_c_tile_lds128<MI, kStoreC, kSystemScope, EPI>(acc, region, rc, row0, col0,
                                                                n_ld - tile_n0, n_ld, alpha, beta,
                                                                rc, 0, bias, epi.act);
        }
        else
            store_split_tile<MI, EPI>(acc, region, rc, row0, col0, N - tile_n0, N, alpha, beta,
                                      tile_split, tile_v, split_plan, bias, epi.act, &s_words[1]);
        if (!more) break;
        // Stores and loads share the vector-memory counter and may complete
        // out of order, so the next tile's first three steps are awaited
        // with everything else; the barrier also ends every wave's epilogue
        // reads of stage 3 before step 3's copies overwrite it.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------
// The four-wave 256 x 256 kernel on the 16 x 16 x 32 matrix instruction
// (v_mfma_f32_16x16x32_bf16): same tile, K step 32, four LDS stages and
// copies three steps ahead, but each wave's 128 x 128 tile is 8 x 8 blocks
// of 16 x 16 (four fp32 accumulators per lane per block, still 256 in all)
// and one MFMA covers a whole K step.  The two instructions do the same work
// per cycle at the same operand bytes per MFMA cycle; on gfx950 the board
// holds a higher clock under a stream of the smaller one.
//
// Fragments (lane l, group g = l / 16): an A fragment is row l % 16 of a
// block, k = 8 g .. 8 g + 7, one 16-byte read (A stage as in the 32 x 32
// kernel); a B fragment is column l % 16, the same k: two transposing reads
// of 4 k rows each.  The 32 lanes of a transposing
// read then cover rows 8 g' + 0..3 for g' in {g, g + 1} (not 4 consecutive
// rows, as in the 32 x 32 kernel), 32 bytes per row; the B swizzle key gains
// a bit from k / 8 (swz_b16) so those 8 rows fall on the 8 different
// 32-byte quarters of a bank line.  The MFMAs take B's fragment first: lane
// l holds row l % 16, columns 4 g .. 4 g + 3 of its block, one 16-byte chunk
// of the epilogue's staging layout.
//
// One set of fragment registers, and a step's 64 MFMAs in two halves: A
// blocks 0 .. 3 with every B block, then A blocks 4 .. 7 with every B block
// (B-major inside a half: MFMA 32 h + 4 jj + i' is block (4 h + i', jj)).
// A fragments 0 .. 3 are then free after MFMA 31, B fragment jj after MFMA
// 35 + 4 jj and A fragments 4 .. 7 after MFMA 63, and each is read again
// for the next step soon after, so the reads spread over the whole step:
//   * first half of step t: the reads of step t's B blocks 6 and 7 and A
//     blocks 4 .. 7, and the last 4 copies of step t + 3, one per 8 MFMAs;
//   * then the wait (step t + 1's copies landed, every read of step t done)
//     and the workgroup barrier;
//   * second half: the reads of step t + 1's A blocks 0 .. 3 and B blocks
//     0 .. 5, each right after its last use (B blocks 6 and 7 wait for the
//     next half: read at the end of this one, they would hold up the next
//     step's first MFMA, which waits for every read of the previous step),
//     and the first 4 copies of step t + 4, one per 8 MFMAs.
// So the reads of stage t run from the barrier of step t - 1 to that of
// step t, and the copies into its stage (for step t + 4) start after the
// barrier that ends those reads.  Spreading the copies over the whole step
// matters more here than with the 32 x 32 instruction: a 16 x 16 MFMA leaves
// the wave a third as many cycles to issue between MFMAs, and a burst of
// copies (all 8 in one half step) kept the texture unit's address queue
// full, stalling the copy instructions and the MFMAs behind them.
__device__ __forceinline__ int swz_b16(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }

template <bool KTAIL, bool EPI, bool TRANSB>
__global__ __launch_bounds__(256, 1) void bf16_q16_kernel(int M, int N, int K, float alpha,
                                                          float beta,
                                                          const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B, float *C,
                                                          int tiles_m, int tiles_n,
                                                          PPSplit split_plan, Epi epi,
                                                          Batch batch) {
    constexpr int BM = 256, BN = 256, S = 4, BK = kPPBK;
    constexpr int WM = 128, WN = 128, MI = 8, NI = 8;  // 16 x 16 blocks per wave
    constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;
    constexpr int A_LOADS = BM / 16 / 4;
    constexpr int B_ROWS = 512 / BN;
    constexpr int B_LOADS = BK / B_ROWS / 4;
    constexpr int COPIES = A_LOADS + B_LOADS;
    constexpr int B_CHUNKS = BN / 8;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S][A_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S][B_STAGE];

    int v, split;
    __shared__ int s_words[2];
    split_tile(blockIdx.x, split_plan, v, split, &s_words[0]);
    const int per_item = tiles_m * tiles_n;
    const int item = v / per_item;
    A += item * batch.stride_a;
    B += item * batch.stride_b;
    C += item * batch.stride_c;
    int tm, tn;
    grouped_tile(v - item * per_item, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int total_steps = (K + BK - 1) / BK;
    const int t_begin = split == 1 ? split_plan.split_step : 0;
    const int t_end = split == 0 ? split_plan.split_step : total_steps;
    const int T = t_end - t_begin;  // this workgroup's steps; t below counts them
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // A copies as in the 32 x 32 kernel.  B copies (B as K x N): copy q of a
    // wave fills rows 8 q + 2 wave + l / 32, whose key differs between even
    // and odd q (bit 3 of the row), so a lane has two source chunks.
    const int a_row_in = lane >> 2;
    const int a_chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t a_off = static_cast<uint32_t>(((16 * wave + a_row_in) * K + 8 * a_chunk) * 2);
    const uint32_t a_step = static_cast<uint32_t>(64 * K * 2);
    const int b_row0 = B_ROWS * wave + lane / B_CHUNKS;
    const int b_c0 = (lane % B_CHUNKS) ^ swz_b16(b_row0);
    const int b_c1 = (lane % B_CHUNKS) ^ swz_b16(b_row0 + 8);
    const bool b_ok0 = (n0 + 8 * b_c0) < N, b_ok1 = (n0 + 8 * b_c1) < N;
    const uint32_t b_off0 = static_cast<uint32_t>((b_row0 * N + 8 * b_c0) * 2);
    const uint32_t b_off1 = static_cast<uint32_t>((b_row0 * N + 8 * b_c1) * 2);
    const uint32_t b_step = static_cast<uint32_t>(4 * B_ROWS * N * 2);
    static_assert(!TRANSB || B_LOADS == A_LOADS, "a transposed B tile copies like A's");

    struct StepCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool a_ok;
    };
    auto step_copy = [&](int t) {
        const int k0 = (t_begin + t) * BK, stage = t % S;
        StepCopy c;
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         (static_cast<long long>(M - m0) * K - k0) * 2);
        if constexpr (TRANSB)
            c.rb = make_desc(B + static_cast<size_t>(n0) * K + k0,
                             (static_cast<long long>(N - n0) * K - k0) * 2);
        else
            c.rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                             (static_cast<long long>(K - k0) * N - n0) * 2);
        c.a_ok = !(KTAIL && k0 + 8 * a_chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 512]);
        c.lb = lds_address(&lds_b[stage][wave * 512]);
        return c;
    };
    auto issue_copy = [&](const StepCopy &c, int q) {
        const int r = q - A_LOADS;
        if (q < A_LOADS)
            lds_dma16(c.ra, c.la + q * 4 * 1024, c.a_ok ? a_off + q * a_step : kOOB);
        else if constexpr (TRANSB)
            lds_dma16(c.rb, c.lb + r * 4 * 1024, c.a_ok ? a_off + r * a_step : kOOB);
        else if (r & 1)
            lds_dma16(c.rb, c.lb + r * 4 * 1024, b_ok1 ? b_off1 + r * b_step : kOOB);
        else
            lds_dma16(c.rb, c.lb + r * 4 * 1024, b_ok0 ? b_off0 + r * b_step : kOOB);
    };

    const int r16 = lane & 15, g = lane >> 4;
    const int a_lane_base = (wm * WM + r16) * BK;
    const int a_pos = (g ^ swz_a32(r16)) * 8;
    const int b_col_lane = wn * WN + 4 * (r16 & 3);
    const int b_row_lane = 8 * g + (r16 >> 2);
    const int bt_lane_base = (wn * WN + r16) * BK;  // TRANSB: row n of the B tile
    bf16x8 fa[MI];
    u32x4 fb[NI];  // filled a dword pair at a time (16-bit inserts cost a wait on the read)
    auto read_a = [&](int stage, int i) {
        const u32x4 x =
            *reinterpret_cast<const u32x4 *>(&lds_a[stage][a_lane_base + 16 * i * BK + a_pos]);
        fa[i] = __builtin_bit_cast(bf16x8, x);
    };
    // B fragment jj: one plain read (TRANSB) or transposing read r of two
    auto read_b = [&](int stage, int jj, int r) {
        if constexpr (TRANSB) {
            fb[jj] = *reinterpret_cast<const u32x4 *>(
                &lds_b[stage][bt_lane_base + 16 * jj * BK + a_pos]);
        } else {
            const int row = 4 * r + b_row_lane;
            const int col = b_col_lane + 16 * jj;
            const int chunk = (col >> 3) ^ swz_b16(row);
            const int elem = row * BN + chunk * 8 + (col & 7);
            const u32x2 part = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (s16x4 __attribute__((address_space(3))) *)&lds_b[stage][elem]));
            fb[jj][2 * r] = part[0];
            fb[jj][2 * r + 1] = part[1];
        }
    };
    constexpr int kBReads = TRANSB ? 1 : 2;  // reads per B fragment

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < NI; ++jj)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][jj][e] = 0.0f;
    constexpr int kHalf = MI * NI / 2;
    auto mfma = [&](int q) {
        const int h = q / kHalf, jj = (q % kHalf) / 4, i = 4 * h + q % 4;
        acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[jj]),
                                                             fa[i], acc[i][jj], 0, 0, 0);
    };
    constexpr int kHalfCopies = COPIES / 2;  // per half step, one per 8 MFMAs
    static_assert(8 * kHalfCopies <= kHalf, "the copies fit a half step");
    constexpr int kWaitSteady = (2 * COPIES & 15) | (7 << 4) | ((2 * COPIES >> 4) << 14);
    constexpr int kWaitDrain = (7 << 4);

    // steps 0 .. 2 and the first half of step 3's copies (which a second
    // half issues in the steady state)
    for (int t = 0; t < S - 1; ++t)
        if (t < T) {
            const StepCopy c = step_copy(t);
#pragma unroll
            for (int q = 0; q < COPIES; ++q) issue_copy(c, q);
        }
    if (T > S - 1) {
        const StepCopy c = step_copy(S - 1);
#pragma unroll
        for (int q = 0; q < kHalfCopies; ++q) issue_copy(c, q);
        __builtin_amdgcn_s_waitcnt(wait_vm(2 * COPIES + kHalfCopies));  // step 0 landed
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitDrain);
    }
    __syncthreads();
    // what a second half reads for the next step, here for step 0 with no
    // MFMA to hide it
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) read_a(0, i);
#pragma unroll
        for (int jj = 0; jj < NI - 2; ++jj)
#pragma unroll
            for (int r = 0; r < kBReads; ++r) read_b(0, jj, r);
    }

    // step t; COPY1: issue the second half of step t + 3's copies, COPY2:
    // the first half of step t + 4's (into the stage step t reads, after the
    // barrier that ends those reads); NEXT: read step t + 1
    auto k_step = [&](int t, auto copy1_tag, auto copy2_tag, auto next_tag) {
        constexpr bool COPY1 = decltype(copy1_tag)::value;
        constexpr bool COPY2 = decltype(copy2_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        const int cur = t % S, nxt = (t + 1) % S;
        StepCopy c;
        if constexpr (COPY1) c = step_copy(t + S - 1);
#pragma unroll
        for (int q = 0; q < kHalf; ++q) {
            mfma(q);
            // B blocks 6 and 7 first (their last uses closed step t - 1),
            // then A blocks 4 .. 7, one per two MFMAs
            if (q < 2 * kBReads) read_b(cur, NI - 2 + q / kBReads, q % kBReads);
            if (q >= 4 && q < 12 && (q & 1) == 0) read_a(cur, 4 + (q - 4) / 2);
            if constexpr (COPY1) {
                if ((q & 7) == 3) issue_copy(c, kHalfCopies + q / 8);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(COPY1 ? kWaitSteady : kWaitDrain);
        __syncthreads();
        StepCopy c2;
        if constexpr (COPY2) c2 = step_copy(t + S);
#pragma unroll
        for (int q = kHalf; q < 2 * kHalf; ++q) {
            mfma(q);
            if constexpr (NEXT) {
                const int u = q - kHalf;  // MFMA u of the second half uses B block u / 4
                if (u < 4) read_a(nxt, u);  // A blocks 0 .. 3: last used in the first half
                if (u % 4 == 3 && u / 4 < NI - 2) {  // B block u / 4: this was its last use
#pragma unroll
                    for (int r = 0; r < kBReads; ++r) read_b(nxt, u / 4, r);
                }
            }
            if constexpr (COPY2) {
                if ((q & 7) == 3) issue_copy(c2, (q - kHalf) / 8);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using On = std::true_type;
    using Off = std::false_type;
    int t = 0;
    for (; t < T - S; ++t) k_step(t, On(), On(), On());  // steps t + 3 and t + 4 exist
    if (t == T - S) {
        k_step(t, On(), Off(), On());
        ++t;
    }
    for (; t < T - 1; ++t) k_step(t, Off(), Off(), On());
    if (T > 0) k_step(T - 1, Off(), Off(), Off());
    // the epilogue stages through the A stages: every wave's last reads are
    // done (the barrier inside the last step), and no copy is in flight

    // epilogue: band i holds block rows 2 i and 2 i + 1; lane l writes row
    // 16 rb + l % 16, chunk 4 jj + l / 16 of each block (rb, jj) of the band
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    static_assert(S * A_STAGE * 2 >= 4 * 16384, "four 16 KB epilogue slices fit in the A stages");
    float *region = reinterpret_cast<float *>(&lds_a[0][0]) + wave * 4096;
    auto write_band = [&](int i, float *reg) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                const int r = 16 * rb + r16, chunk = 4 * jj + g;
                *reinterpret_cast<f32x4 *>(&reg[r * 128 + ((chunk ^ r16) * 4)]) = acc[2 * i + rb][jj];
            }
    };
    const float *bias = EPI && epi.bias ? epi.bias + n0 : nullptr;  // tile's first column
    store_split_bands<MI / 2, EPI>(write_band, region, rc, wm * WM, wn * WN, N - n0, N, alpha, beta,
                                   split, v, split_plan, bias, epi.act, &s_words[1]);
}

const Bf16TileConfig kConfigs[] = {
    {256, 256, "bf16_q4_256x256x32"},
    {256, 128, "bf16_mfma_256x128x64"},
    {128, 256, "bf16_mfma_128x256x64"},
    {128, 128, "bf16_mfma_128x128x64"},
    {256, 256, "bf16_pp_256x256x32"},
    {256, 256, "bf16_q16_256x256x32"},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// Relative per-CU speed of each tile configuration at equal occupancy,
// measured on the square and prefill shapes (the 128 x 128 tile is the
// unit).  At 4096^3 the four-wave 256 x 256 kernel ran 0.5-2.7 us ahead of
// the ping-pong kernel on three boards out of four, and with a split last
// round 1.5-4 us ahead on the four 2048-row prefill shapes.
const double kTileEfficiency[kNumConfigs] = {1.29, 0.85, 0.85, 1.0, 1.27, 1.20};
// LDS bytes per workgroup, which set how many workgroups share a CU.
int tile_lds_bytes(int c) {
    const Bf16TileConfig &t = kConfigs[c];
    return (c == 0 || c == 4 || c == 5) ? 4 * (t.bm + t.bn) * 32 * 2 : 2 * (t.bm + t.bn) * 64 * 2;
}

// ---------------------------------------------------------------------------
// 8-bit float GEMM (E4M3 or E5M2 operands, fp32 accumulation), C = alpha A
// B^T + beta C with B stored N x K: the four-wave 256 x 256 kernel's tile,
// stages and copy pattern at one byte per element.  A K step is 64 elements
// = 64 bytes per row, so the copies, the LDS layout (four 16-byte chunks per
// row, chunk c of row r at c ^ ((r / 4) % 4)) and the LDS bytes read per
// step are those of the bf16 kernel's 32-element step, and B's tile has A's
// shape (no transposing reads).  v_mfma_scale_f32_32x32x64_f8f6f4 (unit
// scales) takes from lane l the 32 bytes k = 32 (l / 32) .. + 31 of row
// (l % 32) for both operands (checked on the device against a host
// product); it does four times the work of the bf16 32x32x16 MFMA at the
// 8-bit rate, so a step is 16 MFMAs per wave instead of 32.  Schedule: the
// fragments the first 8 MFMAs of step t use (two 16-byte reads each) are
// read while the last 8 MFMAs of step t - 1 run, the other two during step
// t's first 8; the copies of step t + 3 go out one per two MFMAs over all
// 16 (a burst of them in half the step was 3.5 % slower); then one wait and
// one barrier, as in the bf16 kernel.  Fragments alternate between two register
// buffers step by step; every step instance is compiled with its buffer and
// its copy flag fixed (see the loop), so the 256 accumulators stay in
// AccVGPRs and nothing spills.
template <bool KTAIL, int FMT>
__global__ __launch_bounds__(256, 1) void fp8_q4_kernel(int M, int N, int K, float alpha,
                                                        float beta,
                                                        const uint8_t *__restrict__ A,
                                                        const uint8_t *__restrict__ B, float *C,
                                                        int tiles_m, int tiles_n,
                                                        PPSplit split_plan) {
    typedef int v8i __attribute__((ext_vector_type(8)));
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    constexpr int BM = 256, BN = 256, S = 4, BK = kFp8BK;  // BK in elements = bytes
    constexpr int WM = 128, WN = 128, MI = 4, NI = 4;
    constexpr int STAGE = BM * BK;                   // bytes, A and B alike
    constexpr int LOADS = BM / 16 / 4;               // 1 KB copies per wave per operand
    constexpr int COPIES = 2 * LOADS;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[S][STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[S][STAGE];

    // tile and K range under the split plan (as the bf16 four-wave kernel)
    int v, split;
    __shared__ int s_words[2];
    split_tile(blockIdx.x, split_plan, v, split, &s_words[0]);
    int tm, tn;
    grouped_tile(v, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int total_steps = (K + BK - 1) / BK;
    const int t_begin = split == 1 ? split_plan.split_step : 0;
    const int t_end = split == 0 ? split_plan.split_step : total_steps;
    const int T = t_end - t_begin;  // this workgroup's steps; t below counts them
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // copies: lane p of a wave writes physical chunk p % 4 of row 16 wave +
    // p / 4 (+ 64 q), holding logical chunk (p % 4) ^ ((p / 16) % 4)
    const int row_in = lane >> 2;
    const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint32_t off0 = static_cast<uint32_t>((16 * wave + row_in) * K + 16 * chunk);
    const uint32_t step64 = static_cast<uint32_t>(64 * K);
    struct StepCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool ok;
    };
    auto step_copy = [&](int t) {
        const int k0 = (t_begin + t) * BK, stage = t % S;
        StepCopy c;
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         static_cast<long long>(M - m0) * K - k0);
        c.rb = make_desc(B + static_cast<size_t>(n0) * K + k0,
                         static_cast<long long>(N - n0) * K - k0);
        c.ok = !(KTAIL && k0 + 16 * chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 1024]);
        c.lb = lds_address(&lds_b[stage][wave * 1024]);
        return c;
    };
    auto issue_copy = [&](const StepCopy &c, int q) {
        const int r = q % LOADS;
        if (q < LOADS)
            lds_dma16(c.ra, c.la + r * 4096, c.ok ? off0 + r * step64 : kOOB);
        else
            lds_dma16(c.rb, c.lb + r * 4096, c.ok ? off0 + r * step64 : kOOB);
    };

    // fragment f of a step: f < MI is A block f, else B block f - MI; read
    // order puts B block 0, the A blocks and B block 1 (what the first eight
    // MFMAs use) first
    const int swz = swz_a32(l32);
    const int p0 = ((2 * h) ^ swz) * 16, p1 = ((2 * h + 1) ^ swz) * 16;
    // each 32-byte fragment is filled by two 16-byte reads into its halves,
    // so it is already one register tuple for the MFMA
    u32x8 fa[2][MI], fb[2][NI];
    auto load16 = [&](const uint8_t *row_base, int half) {
        return *reinterpret_cast<const u32x4 *>(row_base + (half ? p1 : p0));
    };
    // fragment pair `o` (0 .. 7) of a step: B block 0, A blocks 0 .. 3,
    // B blocks 1 .. 3 (the first eight MFMAs use B blocks 0 and 1)
    auto read_pair = [&](int stage, int o, auto buf_tag) {
        constexpr int buf = decltype(buf_tag)::value;
        if (o >= 1 && o <= MI) {
            const int i = o - 1;
            const uint8_t *rb = &lds_a[stage][(wm * WM + 32 * i + l32) * BK];
            fa[buf][i].lo = load16(rb, 0);
            fa[buf][i].hi = load16(rb, 1);
        } else {
            const int jj = o == 0 ? 0 : o - MI;
            const uint8_t *rb = &lds_b[stage][(wn * WN + 32 * jj + l32) * BK];
            fb[buf][jj].lo = load16(rb, 0);
            fb[buf][jj].hi = load16(rb, 1);
        }
    };
    constexpr int kPairs = MI + NI;

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < NI; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
    auto mfma = [&](int q, auto buf_tag) {  // B-major: consecutive MFMAs share B
        constexpr int buf = decltype(buf_tag)::value;
        const int jj = q / MI, i = q % MI;
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_bit_cast(v8i, fb[buf][jj]), __builtin_bit_cast(v8i, fa[buf][i]), acc[i][jj],
            FMT, FMT, 0, 127, 0, 127);
    };
    constexpr int kEarly = 8, kTail = 8;
    // at a step's end the copies of the S - 2 later steps may be in flight
    constexpr int kInFlight = (S - 2) * COPIES;
    static_assert(kInFlight < 64, "vmcnt holds six bits");
    constexpr int kWaitSteady = (kInFlight & 15) | (7 << 4) | ((kInFlight >> 4) << 14);
    constexpr int kWaitDrain = (7 << 4);

    for (int t = 0; t < S - 1; ++t)
        if (t < T) {
            const StepCopy c = step_copy(t);
#pragma unroll
            for (int q = 0; q < COPIES; ++q) issue_copy(c, q);
        }
    if (T >= S - 1)
        __builtin_amdgcn_s_waitcnt(kWaitSteady);
    else
        __builtin_amdgcn_s_waitcnt(kWaitDrain);
    __syncthreads();
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;

    // Each step alternates between the two fragment buffers, and whether it
    // issues copies is a compile-time flag, so every instance of the step
    // below indexes its fragment arrays statically and holds no branch
    // between its MFMAs (a runtime copy flag split the MFMA chains into
    // blocks, and the register allocator then moved an accumulator through
    // VGPRs on every step).  The buffer of step t is (t + copy_end) % 2: the
    // copying steps run in one of two loops, picked once by the parity of
    // copy_end, and both leave the same state for the S - 1 = 3 steps that
    // copy nothing, written out straight (choosing among step variants at
    // run time inside a loop spilled).
    const int copy_end = max(0, T - (S - 1));
    auto k_step = [&](int t, auto buf_tag, auto copy_tag, auto tail_tag) {
        constexpr bool COPY = decltype(copy_tag)::value;
        constexpr bool TAIL = decltype(tail_tag)::value;  // false for step 0 only
        constexpr int buf = decltype(buf_tag)::value;
        const int cur = t % S;
        using Cur = std::integral_constant<int, buf>;
        using Prev = std::integral_constant<int, buf ^ 1>;
        // The fragments the first eight MFMAs use (B blocks 0 and 1, every A
        // block: read pairs 0 .. 5) are read under the previous step's last
        // eight; B blocks 2 and 3 (pairs 6, 7), used only by this step's
        // last eight, under this step's first eight, so that the LDS reads
        // are spread over the whole step instead of half of it.
        // The copies of step t + 3 fill the stage step t - 1 used, whose
        // last fragments were read before the previous barrier: they go out
        // one per two MFMAs over the whole step (a burst of them delays the
        // MFMAs behind the copy queue).
        constexpr int kFirstReads = kPairs - 2;
        StepCopy next;
        if constexpr (COPY) next = step_copy(t + S - 1);
        if constexpr (TAIL) {
#pragma unroll
            for (int q = 0; q < kTail; ++q) {
                mfma(kEarly + q, Prev());
                if (q < kFirstReads) read_pair(cur, q, Cur());
                if constexpr (COPY) {
                    if (q & 1) issue_copy(next, q >> 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {  // step 0: its first fragments are read here, with no MFMA to hide them
#pragma unroll
            for (int q = 0; q < kFirstReads; ++q) read_pair(cur, q, Cur());
        }
#pragma unroll
        for (int q = 0; q < kEarly; ++q) {
            mfma(q, Cur());
            if (q == 1 || q == 4) read_pair(cur, kFirstReads + (q == 4), Cur());
            if constexpr (COPY) {
                if (!TAIL)
                    issue_copy(next, q);
                else if (q & 1)
                    issue_copy(next, COPIES / 2 + (q >> 1));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(COPY ? kWaitSteady : kWaitDrain);
        __syncthreads();
    };
    using On = std::true_type;
    using Off = std::false_type;
    static_assert(S == 4, "three steps follow the last copying step");
    auto last = [&](auto buf_tag) {
#pragma unroll
        for (int q = 0; q < kTail; ++q) {
            mfma(kEarly + q, buf_tag);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (copy_end > 0) {
        int t = 1;
        if (copy_end & 1) {  // step 0 in buffer 1
            k_step(0, Odd(), On(), Off());
            for (; t < copy_end; t += 2) {
                k_step(t, Even(), On(), On());
                k_step(t + 1, Odd(), On(), On());
            }
        } else {  // step 0 in buffer 0, an odd number of copying steps after it
            k_step(0, Even(), On(), Off());
            for (; t + 1 < copy_end; t += 2) {
                k_step(t, Odd(), On(), On());
                k_step(t + 1, Even(), On(), On());
            }
            k_step(t, Odd(), On(), On());
            ++t;
        }
        // t == copy_end, in buffer 0
        k_step(t, Even(), Off(), On());
        k_step(t + 1, Odd(), Off(), On());
        k_step(t + 2, Even(), Off(), On());
        last(Even());
    } else {  // T <= 3: no step issues copies
        k_step(0, Even(), Off(), Off());
        if (T > 1) k_step(1, Odd(), Off(), On());
        if (T > 2) k_step(2, Even(), Off(), On());
        if ((T - 1) & 1)
            last(Odd());
        else
            last(Even());
    }

    // epilogue: as the bf16 kernel's, each wave staging through a private
    // 16 KB slice of the A stages
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    static_assert(S * STAGE >= 4 * 16384, "four 16 KB epilogue slices fit in the A stages");
    float *region = reinterpret_cast<float *>(&lds_a[0][0]) + wave * 4096;
    store_split_tile<MI, false>(acc, region, rc, wm * WM, wn * WN, N - n0, N, alpha, beta, split,
                                v, split_plan, nullptr, kActNone, &s_words[1]);
}

// ---------------------------------------------------------------------------
// The 8-bit float GEMM with a 128-deep K step: the same 256 x 256 tile, four
// waves, 128 x 128 wave tiles and v_mfma_scale_f32_32x32x64_f8f6f4, but each
// step copies 128 bytes of every A and B row, a whole 128-byte line, where
// the 64-deep kernel above copies half lines (64 bytes of each of twice as
// many rows per copy instruction).  Two LDS stages of 64 KB, the whole
// 128 KB: the copies of step t + 1 fill the stage step t - 1 read and are
// issued from the barrier that ends step t - 1 through the first half of
// step t, one per MFMA; the wait at the end of step t takes all of them.
//
// LDS layout: rows of 128 bytes, eight 16-byte chunks, chunk c of row r at
// position c ^ ((r / 2) % 8).  A fragment read (32 x 32 x 64: lane l takes
// row l % 32, bytes 64 s + 32 (l / 32) .. + 31 of the step, s the half step)
// is two 16-byte reads; the 16 lanes of a group read 16 rows at one logical
// chunk, two rows per 256-byte bank line, and the key puts them on 16
// different 16-byte slots; lanes l and l + 16 read the same chunk 16 rows
// apart (same slot, 2 KB apart), which gfx950 serves at full rate.  A copy
// instruction fills 8 rows: lane p takes physical chunk p % 8 of row p / 8.
//
// Schedule of step t (fragment buffer 0 for half step 0, buffer 1 for half
// step 1): the last 8 MFMAs of step t - 1 with the reads of the six
// fragment pairs step t's first 8 MFMAs use; the 16 MFMAs of half step 0
// with the last two pairs of half step 0 and the eight of half step 1; the
// first 8 MFMAs of half step 1; the wait and the barrier.  The 16 copies of
// step t + 1 go out one per MFMA from the start of the step.  Copies past
// the last step are issued with every lane out of range (they write zeros
// into a stage nobody reads), so the loop has no branch around them.
template <bool KTAIL, int FMT>
__global__ __launch_bounds__(256, 1) void fp8_wide_kernel(int M, int N, int K, float alpha,
                                                          float beta,
                                                          const uint8_t *__restrict__ A,
                                                          const uint8_t *__restrict__ B, float *C,
                                                          int tiles_m, int tiles_n,
                                                          PPSplit split_plan) {
    typedef int v8i __attribute__((ext_vector_type(8)));
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    constexpr int BM = 256, BN = 256, S = 2, BK = kFp8WideBK;  // BK in elements = bytes
    constexpr int WM = 128, WN = 128, MI = 4, NI = 4;
    constexpr int STAGE = BM * BK;                   // bytes, A and B alike
    constexpr int LOADS = BM / 8 / 4;                // 1 KB copies per wave per operand
    constexpr int COPIES = 2 * LOADS;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[S][STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[S][STAGE];

    int v, split;
    __shared__ int s_words[2];
    split_tile(blockIdx.x, split_plan, v, split, &s_words[0]);
    int tm, tn;
    grouped_tile(v, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int total_steps = (K + BK - 1) / BK;
    const int t_begin = split == 1 ? split_plan.split_step : 0;
    const int t_end = split == 0 ? split_plan.split_step : total_steps;
    const int T = t_end - t_begin;  // this workgroup's steps; t below counts them
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // copies: lane p of a wave writes physical chunk p % 8 of row 8 wave +
    // p / 8 (+ 32 q), holding logical chunk (p % 8) ^ ((row / 2) % 8)
    const int row_in = lane >> 3;
    const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
    const uint32_t off0 = static_cast<uint32_t>((8 * wave + row_in) * K + 16 * chunk);
    const uint32_t step32 = static_cast<uint32_t>(32 * K);
    struct StepCopy {
        i32x4 ra, rb;
        uint32_t la, lb;
        bool ok;
    };
    auto step_copy = [&](int t) {  // t may be T: then every lane is out of range
        const int k0 = (t_begin + t) * BK, stage = t % S;
        StepCopy c;
        c.ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                         static_cast<long long>(M - m0) * K - k0);
        c.rb = make_desc(B + static_cast<size_t>(n0) * K + k0,
                         static_cast<long long>(N - n0) * K - k0);
        c.ok = t < T && !(KTAIL && k0 + 16 * chunk >= K);
        c.la = lds_address(&lds_a[stage][wave * 1024]);
        c.lb = lds_address(&lds_b[stage][wave * 1024]);
        return c;
    };
    auto issue_copy = [&](const StepCopy &c, int q) {
        const int r = q % LOADS;
        if (q < LOADS)
            lds_dma16(c.ra, c.la + r * 4096, c.ok ? off0 + r * step32 : kOOB);
        else
            lds_dma16(c.rb, c.lb + r * 4096, c.ok ? off0 + r * step32 : kOOB);
    };
    // L2 warm-up: in step t, right after its last copy, every wave loads
    // one 4-byte word from each of its 64 rows of A and of B at step t + 2's
    // k into a scratch LDS area, so that the copies of step t + 2, issued a
    // step later, find their lines in L2 (those copies otherwise wait on
    // HBM at the end of their step).  The step's closing wait leaves these
    // two loads in flight (the counter retires in issue order and they are
    // the last two).  Rows past M or N and k past K are outside the
    // descriptors (no access).
    __shared__ __attribute__((aligned(16))) uint8_t lds_warm[1024];
    const uint32_t warm_lds = lds_address(&lds_warm[0]);
    const uint32_t warm_row = static_cast<uint32_t>((64 * wave + lane) * K);
    auto warm_up = [&](int t) {
        const int k0 = (t_begin + t) * BK;
        const i32x4 da = make_desc(A + static_cast<size_t>(m0) * K + k0,
                                   static_cast<long long>(M - m0) * K - k0);
        const i32x4 db = make_desc(B + static_cast<size_t>(n0) * K + k0,
                                   static_cast<long long>(N - n0) * K - k0);
        const bool ok = t < T;
        lds_dma4_warm(da, warm_lds, ok ? warm_row : kOOB);
        lds_dma4_warm(db, warm_lds, ok ? warm_row : kOOB);
    };

    // fragment reads: half step s, lane half h, read e of a pair takes
    // logical chunk 4 s + 2 h + e
    const int swz = (l32 >> 1) & 7;
    u32x8 fa[2][MI], fb[2][NI];
    auto load16 = [&](const uint8_t *row_base, int s, int e) {
        return *reinterpret_cast<const u32x4 *>(row_base + ((4 * s + 2 * h + e) ^ swz) * 16);
    };
    // fragment pair `o` (0 .. 7) of half step s into buffer s: B block 0, A
    // blocks 0 .. 3, B blocks 1 .. 3 (the first eight MFMAs use B blocks 0
    // and 1)
    auto read_pair = [&](int stage, int s, int o) {
        if (o >= 1 && o <= MI) {
            const int i = o - 1;
            const uint8_t *rb = &lds_a[stage][(wm * WM + 32 * i + l32) * BK];
            fa[s][i].lo = load16(rb, s, 0);
            fa[s][i].hi = load16(rb, s, 1);
        } else {
            const int jj = o == 0 ? 0 : o - MI;
            const uint8_t *rb = &lds_b[stage][(wn * WN + 32 * jj + l32) * BK];
            fb[s][jj].lo = load16(rb, s, 0);
            fb[s][jj].hi = load16(rb, s, 1);
        }
    };
    constexpr int kPairs = MI + NI;

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < NI; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
    auto mfma = [&](int q, int s) {  // B-major: consecutive MFMAs share B
        const int jj = q / MI, i = q % MI;
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_bit_cast(v8i, fb[s][jj]), __builtin_bit_cast(v8i, fa[s][i]), acc[i][jj], FMT,
            FMT, 0, 127, 0, 127);
    };
    constexpr int kMfma = MI * NI;  // per half step
    constexpr int kTail = 8, kEarly = kMfma - kTail;
    constexpr int kFirstReads = kPairs - 2;  // what the first 8 MFMAs of a half step use
    static_assert(COPIES <= kTail + kMfma, "the copies go out before half step 1");
    constexpr int kWaitWarm = wait_vm(2) & ~(15 << 8);  // vmcnt(2), lgkmcnt(0)

    if (T > 0) {
        const StepCopy c = step_copy(0);
#pragma unroll
        for (int q = 0; q < COPIES; ++q) issue_copy(c, q);
    }
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0), lgkmcnt(0)
    __syncthreads();

    // FIRST: step 0, whose first fragments have no previous MFMAs to hide
    // under and which issues all 16 copies of step 1 in its half step 0
    auto k_step = [&](int t, auto first_tag) {
        constexpr bool FIRST = decltype(first_tag)::value;
        const int cur = t % S;
        const StepCopy next = step_copy(t + 1);
        // MFMA slot u = 0 .. 23 of the window from the barrier to the end of
        // half step 0 (the tail, then half step 0) issues copy
        // copy_at(u): two copies per three slots; step 0, with no tail, one
        // per slot of half step 0
        auto copy_at = [](int u) { return FIRST ? u - kTail : (u % 3 == 2 ? -1 : u - u / 3); };
        if constexpr (!FIRST) {
#pragma unroll
            for (int q = 0; q < kTail; ++q) {
                mfma(kEarly + q, 1);
                if (q < kFirstReads) read_pair(cur, 0, q);
                if (copy_at(q) >= 0) issue_copy(next, copy_at(q));
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int q = 0; q < kFirstReads; ++q) read_pair(cur, 0, q);
        }
#pragma unroll
        for (int q = 0; q < kMfma; ++q) {
            mfma(q, 0);
            if (q < 2) read_pair(cur, 0, kFirstReads + q);
            else if (q < 2 + kPairs) read_pair(cur, 1, q - 2);
            const int cq = copy_at(kTail + q);
            if (cq >= 0 && cq < COPIES) issue_copy(next, cq);
            if (cq == COPIES - 1) warm_up(t + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < kEarly; ++q) {
            mfma(q, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's copies of step t + 1 and its reads (the two warm-up
        // loads may stay in flight)
        __builtin_amdgcn_s_waitcnt(kWaitWarm);
        __syncthreads();
    };
    if (T > 0) k_step(0, std::true_type());
    for (int t = 1; t < T; ++t) k_step(t, std::false_type());
    __builtin_amdgcn_s_waitcnt(7 << 4);  // the last warm-up loads
    if (T > 0) {
#pragma unroll
        for (int q = 0; q < kTail; ++q) {
            mfma(kEarly + q, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // epilogue: as the bf16 kernel's, each wave staging through a private
    // 16 KB slice of the A stages (the last barrier ended every read, and
    // the last step's copies were all out of range)
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    static_assert(S * STAGE >= 4 * 16384, "four 16 KB epilogue slices fit in the A stages");
    float *region = reinterpret_cast<float *>(&lds_a[0][0]) + wave * 4096;
    store_split_tile<MI, false>(acc, region, rc, wm * WM, wn * WN, N - n0, N, alpha, beta, split,
                                v, split_plan, nullptr, kActNone, &s_words[1]);
}

// Calls f(ktail, epi) with the two flags as std::integral_constant values, so
// that a launcher can pick one of its four kernel instantiations.
template <class F>
void with_flags(bool ktail, bool epi, F &&f) {
    if (ktail) {
        if (epi) f(std::true_type(), std::true_type());
        else f(std::true_type(), std::false_type());
    } else {
        if (epi) f(std::false_type(), std::true_type());
        else f(std::false_type(), std::false_type());
    }
}

// Checks a split plan against the tile count and K; fills `plan` (whole
// tiles only when split is null).
bool make_plan(const PPSplit *split, long long tiles, int K, PPSplit &plan, int bk = kPPBK) {
    plan = PPSplit{static_cast<int>(tiles), 0, nullptr, nullptr, nullptr, 0u, 0,
                   static_cast<int>(tiles), 0, nullptr};
    if (split == nullptr) return true;
    const int steps = (K + bk - 1) / bk;
    if (split->split_from < 0 || split->split_from > tiles || split->split_step < 1 ||
        split->split_step >= steps || split->poll_limit < 0 ||
        (split->split_from < tiles && (split->partials == nullptr || split->flags == nullptr ||
                                       split->claims == nullptr)) ||
        (split->xcd_pairs && (tiles - split->split_from) % 8 != 0))
        return false;
    plan = *split;
    plan.grid_tiles = static_cast<int>(tiles);
    return true;
}

// persist_grid > 0 (the 32 x 32 kernel, batched calls only): a persistent
// grid of that many workgroups, a multiple of 8, when there are more tiles.
template <bool Q16>
hipError_t launch_q4(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                     const uint16_t *B, float *C, const PPSplit *split, const Epi &epi,
                     hipStream_t stream, const Batch &batch = kOneItem, bool trans_b = false,
                     int persist_grid = 0) {
    const long long tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
    const long long tiles = tiles_m * tiles_n;
    const long long total = tiles * batch.items;
    if (total > 0x3fffffffLL || batch.items < 1 || (batch.items > 1 && split != nullptr))
        return hipErrorInvalidValue;
    if (persist_grid < 0 || persist_grid % 8 != 0 ||
        (persist_grid > 0 && (Q16 || split || epi_on(epi))))
        return hipErrorInvalidValue;
    PPSplit plan;
    if (!make_plan(split, total, K, plan)) return hipErrorInvalidValue;
    const bool persist = persist_grid > 0 && total > persist_grid;
    const long long grid = persist ? persist_grid : plan.split_from + 2 * (total - plan.split_from);
    auto go = [&](auto ktail, auto e, auto tb) {
        constexpr bool KT = decltype(ktail)::value, EP = decltype(e)::value,
                       TB = decltype(tb)::value;
        const dim3 g(static_cast<unsigned>(grid));
        if constexpr (Q16)
            bf16_q16_kernel<KT, EP, TB><<<g, dim3(kThreads), 0, stream>>>(
                M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m),
                static_cast<int>(tiles_n), plan, epi, batch);
        else if (!EP && persist)  // batched calls carry no fused epilogue
            bf16_q4_kernel<KT, false, TB, true><<<g, dim3(kThreads), 0, stream>>>(
                M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m),
                static_cast<int>(tiles_n), plan, epi, batch);
        else
            bf16_q4_kernel<KT, EP, TB><<<g, dim3(kThreads), 0, stream>>>(
                M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m),
                static_cast<int>(tiles_n), plan, epi, batch);
    };
    if (trans_b) {
        if (epi_on(epi)) return hipErrorInvalidValue;  // no fused epilogue in batched calls
        if (K % kPPBK != 0) go(std::true_type(), std::false_type(), std::true_type());
        else go(std::false_type(), std::false_type(), std::true_type());
    } else {
        with_flags(K % kPPBK != 0, epi_on(epi),
                   [&](auto ktail, auto e) { go(ktail, e, std::false_type()); });
    }
    return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_cfg(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                      const uint16_t *B, float *C, const Epi &epi, hipStream_t stream,
                      const Batch &batch = kOneItem, bool trans_b = false, bool staged = false) {
    const long long tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const long long tiles = tiles_m * tiles_n * batch.items;
    if (tiles > 0x7fffffffLL || batch.items < 1) return hipErrorInvalidValue;
    if ((trans_b || staged) && (epi_on(epi) || BM != 128 || BN != 128))
        return hipErrorInvalidValue;  // batched 128 x 128 calls only
    const dim3 grid(static_cast<unsigned>(tiles)), block(kThreads);
    const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
    if constexpr (BM == 128 && BN == 128) {
        if (trans_b || staged) {
            auto go = [&](auto kt, auto tb, auto st) {
                bf16_mfma_kernel<BM, BN, decltype(kt)::value, false, decltype(tb)::value,
                                 decltype(st)::value>
                    <<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn, epi,
                                                 batch);
            };
            auto with_st = [&](auto kt, auto tb) {
                if (staged) go(kt, tb, std::true_type());
                else go(kt, tb, std::false_type());
            };
            auto with_tb = [&](auto kt) {
                if (trans_b) with_st(kt, std::true_type());
                else with_st(kt, std::false_type());
            };
            if (K % kBK != 0) with_tb(std::true_type());
            else with_tb(std::false_type());
            return hipGetLastError();
        }
    }
    with_flags(K % kBK != 0, epi_on(epi), [&](auto ktail, auto e) {
        bf16_mfma_kernel<BM, BN, decltype(ktail)::value, decltype(e)::value>
            <<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn, epi, batch);
    });
    return hipGetLastError();
}

// Batched calls with B as K x N and no fused epilogue on S LDS stages (copies
// S - 1 K steps ahead), C stored straight from the accumulators or through
// LDS (staged).
template <int BM, int BN, int S>
hipError_t launch_deep(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                       const uint16_t *B, float *C, hipStream_t stream, const Batch &batch,
                       bool staged) {
    const long long tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const long long tiles = tiles_m * tiles_n * batch.items;
    if (tiles > 0x7fffffffLL || batch.items < 1) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tiles)), block(kThreads);
    const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
    auto go = [&](auto kt, auto st) {
        bf16_mfma_kernel<BM, BN, decltype(kt)::value, false, false, decltype(st)::value, S>
            <<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn, kNoEpi, batch);
    };
    auto with_st = [&](auto kt) {
        if (staged) go(kt, std::true_type());
        else go(kt, std::false_type());
    };
    if (K % kBK != 0) with_st(std::true_type());
    else with_st(std::false_type());
    return hipGetLastError();
}

template <int BM, int BN, int S>
hipError_t launch_pp(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                     const uint16_t *B, float *C, const PPSplit *split, const Epi &epi,
                     hipStream_t stream) {
    const long long tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x3fffffffLL) return hipErrorInvalidValue;
    PPSplit plan;
    if (!make_plan(split, tiles, K, plan)) return hipErrorInvalidValue;
    const long long grid = plan.split_from + 2 * (tiles - plan.split_from);
    with_flags(K % kPPBK != 0, epi_on(epi), [&](auto ktail, auto e) {
        bf16_pp_kernel<BM, BN, S, decltype(ktail)::value, decltype(e)::value>
            <<<dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream>>>(
                M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m),
                static_cast<int>(tiles_n), plan, epi);
    });
    return hipGetLastError();
}

}  // namespace

int bf16_num_tile_configs() { return kNumConfigs; }

const Bf16TileConfig &bf16_tile_config(int cfg) { return kConfigs[cfg]; }

int bf16_pp_config() { return 4; }

bool bf16_config_splits(int cfg) { return cfg == 0 || cfg == 4 || cfg == 5; }

const char *bf16_split_name(int cfg, bool xcd_pairs) {
    switch (cfg) {
        case 4: return xcd_pairs ? "bf16_pp_256x256x32_splitk_xcd" : "bf16_pp_256x256x32_splitk";
        case 5: return xcd_pairs ? "bf16_q16_256x256x32_splitk_xcd" : "bf16_q16_256x256x32_splitk";
        default: return xcd_pairs ? "bf16_q4_256x256x32_splitk_xcd" : "bf16_q4_256x256x32_splitk";
    }
}

int bf16_pp_split_tiles(int M, int N, int K, int num_cus) {
    // Split the last round when it is at most half full and each half of K
    // keeps at least four steps.
    const long long tiles =
        static_cast<long long>((M + kPPTile - 1) / kPPTile) * ((N + kPPTile - 1) / kPPTile);
    const long long r = num_cus > 0 ? tiles % num_cus : 0;
    const int steps = (K + kPPBK - 1) / kPPBK;
    if (r == 0 || 2 * r > num_cus || steps < 8) return 0;
    return static_cast<int>(r);
}

int bf16_pick_tile_config(int M, int N, int K, int num_cus, bool allow_split) {
    // Estimated time = rounds x (workgroups sharing a CU) x tile area /
    // efficiency, where a partial last round counts half plus its filled
    // fraction (a half-empty round runs faster per tile: less contention).
    const int lds_per_cu = 160 * 1024;
    int best = 0;
    double best_cost = 0.0;
    for (int c = 0; c < kNumConfigs; ++c) {
        const int bm = kConfigs[c].bm, bn = kConfigs[c].bn;
        const long long wgs = static_cast<long long>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        const int occ = lds_per_cu / tile_lds_bytes(c);
        const long long slots = static_cast<long long>(num_cus) * occ;
        const long long full = wgs / slots, rem = wgs % slots;
        double rounds =
            static_cast<double>(full) + (rem ? 0.5 + 0.5 * static_cast<double>(rem) / slots : 0.0);
        // a split last round (either 256 x 256 kernel): half the K steps on
        // twice the CUs, plus the exchange of partial tiles
        if (allow_split && bf16_config_splits(c) && bf16_pp_split_tiles(M, N, K, num_cus) > 0)
            rounds = static_cast<double>(full) + 0.6;
        const double cost = rounds * occ * bm * bn / kTileEfficiency[c];
        if (c == 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

hipError_t launch_fp8_gemm(int M, int N, int K, float alpha, float beta, const uint8_t *A,
                           const uint8_t *B, float *C, int fmt, const PPSplit *split,
                           hipStream_t stream, bool wide) {
    const long long tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x3fffffffLL || (fmt != 0 && fmt != 1) || K % 16 != 0)
        return hipErrorInvalidValue;
    const int bk = wide ? kFp8WideBK : kFp8BK;
    PPSplit plan;
    if (!make_plan(split, tiles, K, plan, bk)) return hipErrorInvalidValue;
    const long long grid = plan.split_from + 2 * (tiles - plan.split_from);
    const dim3 g(static_cast<unsigned>(grid)), block(kThreads);
    const bool ktail = K % bk != 0;
    const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
    auto go = [&](auto kt, auto f) {
        constexpr bool KT = decltype(kt)::value;
        constexpr int F = decltype(f)::value;
        if (wide)
            fp8_wide_kernel<KT, F><<<g, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn,
                                                            plan);
        else
            fp8_q4_kernel<KT, F><<<g, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn,
                                                          plan);
    };
    using F0 = std::integral_constant<int, 0>;
    using F1 = std::integral_constant<int, 1>;
    if (fmt == 0) {
        if (ktail) go(std::true_type(), F0());
        else go(std::false_type(), F0());
    } else {
        if (ktail) go(std::true_type(), F1());
        else go(std::false_type(), F1());
    }
    return hipGetLastError();
}

int fp8_split_tiles(int M, int N, int K, int num_cus, int bk) {
    // as for bf16: split the last round when it is at most half full and
    // each half keeps at least four K steps
    const long long tiles =
        static_cast<long long>((M + kPPTile - 1) / kPPTile) * ((N + kPPTile - 1) / kPPTile);
    const long long r = num_cus > 0 ? tiles % num_cus : 0;
    const int steps = (K + bk - 1) / bk;
    if (r == 0 || 2 * r > num_cus || steps < 8) return 0;
    return static_cast<int>(r);
}

hipError_t launch_bf16_batched(int cfg, int M, int N, int K, float alpha, float beta,
                               const uint16_t *A, const uint16_t *B, float *C, const Batch &batch,
                               bool trans_b, hipStream_t stream, bool staged, int persist_grid,
                               int stages) {
    if (persist_grid != 0 && cfg != 0) return hipErrorInvalidValue;
    if (stages != 2) {
        if (trans_b) return hipErrorInvalidValue;
        if (cfg == 3 && stages == 4)
            return launch_deep<128, 128, 4>(M, N, K, alpha, beta, A, B, C, stream, batch, staged);
        if (cfg == 1 && stages == 3)
            return launch_deep<256, 128, 3>(M, N, K, alpha, beta, A, B, C, stream, batch, staged);
        return hipErrorInvalidValue;
    }
    switch (cfg) {
        case 0:
            return launch_q4<false>(M, N, K, alpha, beta, A, B, C, nullptr, kNoEpi, stream, batch,
                                    trans_b, persist_grid);
        case 5:
            return launch_q4<true>(M, N, K, alpha, beta, A, B, C, nullptr, kNoEpi, stream, batch,
                                   trans_b);
        case 3:
            return launch_cfg<128, 128>(M, N, K, alpha, beta, A, B, C, kNoEpi, stream, batch,
                                        trans_b, staged);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bf16_mfma(int cfg, int M, int N, int K, float alpha, float beta,
                            const uint16_t *A, const uint16_t *B, float *C, const PPSplit *split,
                            const Epi &epi, hipStream_t stream) {
    if (split != nullptr && !bf16_config_splits(cfg)) return hipErrorInvalidValue;
    switch (cfg) {
        case 0: return launch_q4<false>(M, N, K, alpha, beta, A, B, C, split, epi, stream);
        case 5: return launch_q4<true>(M, N, K, alpha, beta, A, B, C, split, epi, stream);
        case 1: return launch_cfg<256, 128>(M, N, K, alpha, beta, A, B, C, epi, stream);
        case 2: return launch_cfg<128, 256>(M, N, K, alpha, beta, A, B, C, epi, stream);
        case 3: return launch_cfg<128, 128>(M, N, K, alpha, beta, A, B, C, epi, stream);
        case 4:
            return launch_pp<kPPTile, kPPTile, 4>(M, N, K, alpha, beta, A, B, C, split, epi,
                                                  stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mgemm
