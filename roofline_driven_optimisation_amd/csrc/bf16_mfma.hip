// bf16-input, fp32-accumulate GEMM on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), LDS-tiled and double-buffered.
//
// Structure (page "Naive GEMM and Roofline analysis", section 10.4, the three
// tile levels plus double buffering):
//   * workgroup tile BM x BN (256 or 128 each), K step 64, 256 threads = four
//     64-lane waves in 2 x 2, each owning a (BM/2) x (BN/2) sub-tile built from
//     32 x 32 MFMA blocks; a 128 x 128 wave tile keeps 256 fp32 accumulators
//     per lane, which is what makes the LDS traffic per MFMA small enough;
//   * the next K tile is fetched into registers (16-byte loads, coalesced
//     along the contiguous dimension) while the current tile's MFMAs run, and
//     written to the other LDS buffer afterwards: one barrier per K step
//     (page "Where kernel performance comes from", overlap section);
//   * fused alpha/beta epilogue in fp32; C is not read when beta == 0.
//
// Operand layout.  Both MFMA operands want eight k-consecutive bf16 values
// per lane (row l % 32 of A, column l % 32 of B, k-octet l / 32).  A is
// k-contiguous in memory and is copied as is.  B is n-contiguous, so each
// thread loads an 8 x 8 (or 4 x 8) k-by-n block of B with 16-byte loads and
// transposes it in registers before writing it to LDS as B^T[n][k]; the
// transpose costs a few ALU ops per element and keeps every LDS access a
// 16-byte access.
//
// LDS rows are 64 bf16 = 128 bytes = eight 16-byte chunks.  Chunk c of row r
// is stored at position c ^ (r % 8) (an XOR swizzle, the software form of the
// swizzled shared-memory layouts of page "Memory hierarchy and cost table",
// section 4.3.4), so the eight rows read by any eight consecutive lanes land
// in eight different bank groups for both the fragment reads and the tile
// writes.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kChunksPerRow = kBK / 8;  // 16-byte chunks per 64-element LDS row

template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
    static constexpr int MI = WM / 32, NI = WN / 32; // MFMA blocks per wave
    static constexpr int A_CHUNKS = BM * kChunksPerRow / kThreads;  // A chunks per thread
    static constexpr int KR = BN / 32;                // k-rows per B block per thread
    static constexpr int KB = kBK / KR;               // B blocks along k
    static_assert(KR == 8 || KR == 4, "B block height must be 8 or 4");
    static_assert(KB * (BN / 8) == kThreads, "one B block per thread");
    static constexpr int LDS_BYTES = 2 * (BM + BN) * kBK * 2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void bf16_mfma_kernel(int M, int N, int K, float alpha,
                                                                float beta,
                                                                const uint16_t *__restrict__ A,
                                                                const uint16_t *__restrict__ B,
                                                                float *C, int tiles_m,
                                                                int tiles_n) {
    using T = Tile<BM, BN>;
    __shared__ u32x4 As[2][BM * kChunksPerRow];
    __shared__ u32x4 Bt[2][BN * kChunksPerRow];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // A staging: chunk i of this thread is row tid / 8 + 32 i, k-chunk tid % 8.
    // B staging: one KR x 8 block, k-rows kb*KR .. kb*KR+KR-1, columns nb*8 .. nb*8+7.
    const int a_kc = tid & 7;
    const int b_kb = tid % T::KB, b_nb = tid / T::KB;
    u32x4 ra[T::A_CHUNKS], rb[T::KR];

    auto load_tile = [&](int k0) {
        const int ka = k0 + a_kc * 8;
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int row = m0 + (tid >> 3) + 32 * i;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < M && ka < K)
                v = *reinterpret_cast<const u32x4 *>(A + static_cast<size_t>(row) * K + ka);
            ra[i] = v;
        }
        const int n = n0 + b_nb * 8;
#pragma unroll
        for (int e = 0; e < T::KR; ++e) {
            const int kr = k0 + b_kb * T::KR + e;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (kr < K && n < N)
                v = *reinterpret_cast<const u32x4 *>(B + static_cast<size_t>(kr) * N + n);
            rb[e] = v;
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int r = (tid >> 3) + 32 * i;
            As[buf][r * kChunksPerRow + (a_kc ^ (r & 7))] = ra[i];
        }
        // Transpose the KR x 8 block: column j of the block becomes KR
        // k-consecutive bf16 values of row n = nb*8 + j of B^T.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int d = j >> 1;
            const int nl = b_nb * 8 + j;
            if (T::KR == 8) {
                u32x4 col;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    col[q] = (j & 1) ? pack_hi(rb[2 * q][d], rb[2 * q + 1][d])
                                     : pack_lo(rb[2 * q][d], rb[2 * q + 1][d]);
                Bt[buf][nl * kChunksPerRow + (b_kb ^ (nl & 7))] = col;
            } else {
                u32x2 col;
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    col[q] = (j & 1) ? pack_hi(rb[2 * q][d], rb[2 * q + 1][d])
                                     : pack_lo(rb[2 * q][d], rb[2 * q + 1][d]);
                // four k values = half a chunk: chunk b_kb / 2, half b_kb % 2
                u32x2 *half = reinterpret_cast<u32x2 *>(&Bt[buf][0]);
                half[(nl * kChunksPerRow + ((b_kb >> 1) ^ (nl & 7))) * 2 + (b_kb & 1)] = col;
            }
        }
    };

    f32x16 acc[T::MI][T::NI];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int ktiles = (K + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    // Fragment rows of this lane are wm*WM + 32 i + l32 (A) and
    // wn*WN + 32 j + l32 (B^T); both are congruent to lane mod 8, which is
    // therefore the swizzle key of every fragment read.
    const int swz = lane & 7;
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ktiles) load_tile((t + 1) * kBK);
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int pos = (2 * s + h) ^ swz;
            bf16x8 a[T::MI], b[T::NI];
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
                a[i] = as_bf16x8(As[cur][(wm * T::WM + 32 * i + l32) * kChunksPerRow + pos]);
#pragma unroll
            for (int j = 0; j < T::NI; ++j)
                b[j] = as_bf16x8(Bt[cur][(wn * T::WN + 32 * j + l32) * kChunksPerRow + pos]);
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int j = 0; j < T::NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < ktiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: register r of a 32 x 32 block is row 8*(r/4) + 4*(lane/32) + r%4,
    // column lane % 32.
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NI; ++j) {
            const int col = n0 + wn * T::WN + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * T::WM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M && col < N) {
                    const size_t idx = static_cast<size_t>(row) * N + col;
                    float out = alpha * acc[i][j][r];
                    if (beta != 0.0f) out = fmaf(beta, C[idx], out);
                    C[idx] = out;
                }
            }
        }
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
    bf16_mfma_kernel<BM, BN><<<dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, stream>>>(
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
