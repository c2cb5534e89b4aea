// bf16-input, fp32-accumulate GEMM on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), LDS-tiled and double-buffered.
//
// Structure (page "Naive GEMM and Roofline analysis", section 10.4, the three
// tile levels plus double buffering):
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
//   * fused alpha/beta epilogue in fp32; C is not read when beta == 0.
//
// Edges.  The buffer resource's range check turns every out-of-range load
// into zeros and drops every out-of-range store; a column or k index past the
// matrix (which would otherwise wrap into the next row) is redirected to an
// out-of-range offset.  The main loop has no branches on the shape.
//
// Operand layouts in LDS (rows of 16-byte chunks, XOR-swizzled, the software
// form of the swizzled layouts of page "Memory hierarchy and cost table",
// section 4.3.4):
//   * A tile: BM rows of 64 k (128 bytes, 8 chunks); chunk c of row r sits at
//     position c ^ (r % 8).  A fragment (row l % 32, k-octet l / 32) is one
//     ds_read_b128, and any 8 consecutive lanes hit 8 different bank groups.
//   * B tile: 64 k-rows of BN n (natural row-major); chunk c of row k sits at
//     position c ^ swz_b(k).  The B fragment needs 8 k-consecutive values of
//     one column per lane; ds_read_b64_tr_b16 provides exactly that transpose:
//     within a 16-lane group, lane i receives element i % 4 of the 8 bytes
//     read by lanes 4e + i / 4 (e = 0..3).  So if lane j reads the 4 columns
//     n0 + 4 (j % 4) .. +3 of row k0 + j / 4, lane i gets rows k0 .. k0+3 of
//     column n0 + i; two such reads give the 8 k values of a fragment.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
// An offset past every descriptor range (all ranges are clamped below 2^31).
// Buffer builtins take the offset as int: always pass static_cast<int>(...).
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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

// Swizzle key of B row k: the four rows read by one 16-lane group of a
// transposed read land in four different 32-byte bank groups.  It depends on
// k % 4 only, so a lane's read address changes by plain immediate offsets
// across rows and k16 sub-steps.
__device__ __forceinline__ int swz_b(int k) { return (k & 3) << 1; }

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
// of the buffer `desc` into LDS at `lds_addr` + 16 * lane.  Written as inline
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
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(desc)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p));
}

template <int BM, int BN, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void bf16_mfma_kernel(int M, int N, int K, float alpha,
                                                                float beta,
                                                                const uint16_t *__restrict__ A,
                                                                const uint16_t *__restrict__ B,
                                                                float *C, int tiles_m,
                                                                int tiles_n) {
    using T = Tile<BM, BN>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][T::A_STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][T::B_STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // ---- per-lane global offsets of this wave's direct-to-LDS loads --------
    // A load L = wave + 4 i covers tile rows 8L .. 8L+7; lane p fills chunk
    // position p % 8 of row 8L + p / 8 with logical chunk (p % 8) ^ (p / 8).
    const int a_row_in = lane >> 3;
    const int a_chunk = (lane & 7) ^ a_row_in;
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

    auto issue_tile = [&](int k0, int stage) {
        // descriptors based at the tile origin
        const i32x4 ra = make_desc(A + static_cast<size_t>(m0) * K + k0,
                                   (static_cast<long long>(M - m0) * K - k0) * 2);
        const i32x4 rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                                   (static_cast<long long>(K - k0) * N - n0) * 2);
        const bool a_ok = !(KTAIL && k0 + 8 * a_chunk >= K);
        const uint32_t la = lds_address(&lds_a[stage][wave * 512]);
        const uint32_t lb = lds_address(&lds_b[stage][wave * 512]);
#pragma unroll
        for (int i = 0; i < T::A_LOADS; ++i)
            lds_dma16(ra, la + i * 4 * 1024, a_ok ? a_off + i * a_step : kOOB);
#pragma unroll
        for (int i = 0; i < T::B_LOADS; ++i)
            lds_dma16(rb, lb + i * 4 * 1024, b_ok ? b_off + i * b_step : kOOB);
    };

    // ---- fragment reads ----------------------------------------------------
    // A: row wm*WM + 32 i + l32, chunk 2 s + h at position chunk ^ (lane % 8).
    // B: lane's transposed-read address: row 16 s + 8 h' + 4 r + j / 4 and
    //    columns n_frag + 4 (j % 4), where j = lane % 16, h' = (lane / 32).
    const int a_lane_base = (wm * T::WM + l32) * kBK;
    const int g = lane >> 4, j16 = lane & 15;
    const int b_col_lane = wn * T::WN + 16 * (g & 1) + 4 * (j16 & 3);  // + 32 j
    const int b_row_lane = 8 * (g >> 1) + (j16 >> 2);                  // + 16 s + 4 r

    auto read_frags = [&](int stage, int s, bf16x8 (&a)[T::MI], bf16x8 (&b)[T::NI]) {
        const uint16_t *sa = lds_a[stage];
        const uint16_t *sb = lds_b[stage];
        const int pos = ((2 * s + h) ^ (lane & 7)) * 8;
#pragma unroll
        for (int i = 0; i < T::MI; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                &sa[a_lane_base + 32 * i * kBK + pos]);
            a[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj) {
            s16x4 part[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int row = 16 * s + 4 * r + b_row_lane;
                const int col = b_col_lane + 32 * jj;
                const int chunk = (col >> 3) ^ swz_b(row);
                const int elem = row * BN + chunk * 8 + (col & 7);
                part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)&sb[elem]);
            }
            const s16x4 lo = part[0], hi = part[1];
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            b[jj] = __builtin_bit_cast(bf16x8, both);
        }
    };

    f32x16 acc[T::MI][T::NI];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;

    const int ktiles = (K + kBK - 1) / kBK;
    issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Software pipeline of one K step (tile t in stage t % 2):
    //   issue direct loads of tile t+1 into the other stage
    //   sub-steps 0..2: read fragments of sub-step s+1, 16 MFMAs of sub-step s
    //   sub-step 3:     wait for own loads + barrier (the current stage is
    //                   then no longer read and tile t+1 is complete), read
    //                   tile t+1's sub-step-0 fragments, 16 MFMAs of sub-step 3
    // Past the last tile the "next" tile lies beyond K, so its loads are all
    // out of range and only write zeros into the idle stage.  Scheduling
    // barriers keep each sub-step's fragment reads (and the step's global
    // loads) interleaved with its MFMAs.
    bf16x8 fa[2][T::MI], fb[2][T::NI];
    read_frags(0, 0, fa[0], fb[0]);
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        issue_tile((t + 1) * kBK, cur ^ 1);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int f = s & 1;
            if (s + 1 < kBK / 16) {
                read_frags(cur, s + 1, fa[f ^ 1], fb[f ^ 1]);
            } else {
                __builtin_amdgcn_s_waitcnt(0);  // own loads of tile t+1 landed, reads done
                __syncthreads();
                read_frags(cur ^ 1, 0, fa[f ^ 1], fb[f ^ 1]);
            }
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int jj = 0; jj < T::NI; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][i], fb[f][jj],
                                                                        acc[i][jj], 0, 0, 0);
            constexpr int kReads = T::MI + 2 * T::NI;
#pragma unroll
            for (int q = 0; q < T::MI * T::NI; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // one MFMA
                if (q < kReads) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // one LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- epilogue: register r of a 32 x 32 block is row 8*(r/4) + 4*h + r%4,
    // column l32; rows past M fall outside the descriptor, columns past N are
    // redirected out of range.
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + static_cast<size_t>(m0) * N + n0,
                  (static_cast<long long>(M - m0) * N - n0) * 4);
    auto epilogue = [&](const bool read_c) {
#pragma unroll
        for (int jj = 0; jj < T::NI; ++jj) {
            const int col = wn * T::WN + 32 * jj + l32;
            const bool col_ok = (n0 + col) < N;
#pragma unroll
            for (int i = 0; i < T::MI; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * T::WM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    const uint32_t off =
                        col_ok ? static_cast<uint32_t>((row * N + col) * 4) : kOOB;
                    float out = alpha * acc[i][jj][r];
                    if (read_c) {
                        const float cin = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(off), 0, 0));
                        out = fmaf(beta, cin, out);
                    }
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), rc,
                                                          static_cast<int>(off), 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);  // one block at a time: bounded registers
            }
        }
    };
    epilogue(beta != 0.0f);
}

const Bf16TileConfig kConfigs[] = {
    {256, 256, "bf16_mfma_256x256x64"},
    {256, 128, "bf16_mfma_256x128x64"},
    {128, 256, "bf16_mfma_128x256x64"},
    {128, 128, "bf16_mfma_128x128x64"},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// Relative MFMA efficiency assumed for each tile (LDS bytes per MFMA grow as
// the wave tile shrinks).
const double kTileEfficiency[kNumConfigs] = {1.0, 0.85, 0.85, 0.5};

template <int BM, int BN>
hipError_t launch_cfg(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                      const uint16_t *B, float *C, hipStream_t stream) {
    const long long tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tiles)), block(kThreads);
    if (K % kBK == 0)
        bf16_mfma_kernel<BM, BN, false><<<grid, block, 0, stream>>>(
            M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m), static_cast<int>(tiles_n));
    else
        bf16_mfma_kernel<BM, BN, true><<<grid, block, 0, stream>>>(
            M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_m), static_cast<int>(tiles_n));
    return hipGetLastError();
}

}  // namespace

int bf16_num_tile_configs() { return kNumConfigs; }

const Bf16TileConfig &bf16_tile_config(int cfg) { return kConfigs[cfg]; }

int bf16_pick_tile_config(int M, int N, int K, int num_cus) {
    (void)K;
    const int lds_per_cu = 160 * 1024;
    int best = 0;
    double best_cost = 0.0;
    for (int c = 0; c < kNumConfigs; ++c) {
        const int bm = kConfigs[c].bm, bn = kConfigs[c].bn;
        const long long wgs = static_cast<long long>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        const int lds = 2 * (bm + bn) * kBK * 2;
        const long long slots = static_cast<long long>(num_cus) * (lds_per_cu / lds);
        const long long rounds = (wgs + slots - 1) / slots;
        const double cost = static_cast<double>(rounds) * bm * bn / kTileEfficiency[c];
        if (c == 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

hipError_t launch_bf16_mfma(int cfg, int M, int N, int K, float alpha, float beta,
                            const uint16_t *A, const uint16_t *B, float *C, hipStream_t stream) {
    switch (cfg) {
        case 0: return launch_cfg<256, 256>(M, N, K, alpha, beta, A, B, C, stream);
        case 1: return launch_cfg<256, 128>(M, N, K, alpha, beta, A, B, C, stream);
        case 2: return launch_cfg<128, 256>(M, N, K, alpha, beta, A, B, C, stream);
        case 3: return launch_cfg<128, 128>(M, N, K, alpha, beta, A, B, C, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mgemm
