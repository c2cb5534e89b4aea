// fp32 GEMM on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), LDS-tiled.
// Two kernels share the tiling below: f32_dma_kernel (further down; direct
// global -> LDS copies, the path for 16-byte aligned rows) and
// f32_mfma_kernel (register-staged copies, any alignment and any size).
//
// Structure (page "Naive GEMM and Roofline analysis", section 10.4: block
// tile -> warp tile -> matrix instruction, with double buffering):
//   * workgroup tile 128 x 128, K step 32, 256 threads = 4 waves of 64 lanes
//     in a 2 x 2 arrangement, each wave owning a 64 x 64 sub-tile made of
//     2 x 2 MFMA blocks of 32 x 32;
//   * A and B tiles are staged through two LDS buffers; the next tile's
//     global loads are issued into registers before the current tile's MFMAs
//     and written to the other buffer afterwards, so one barrier per K step
//     suffices (page "Where kernel performance comes from", overlap section:
//     load k+1 while computing k);
//   * the fused epilogue applies alpha and beta in fp32 and never reads C when
//     beta == 0.
//
// gfx950 has no reduced-precision fp32 matrix path to fall into: products and
// sums stay fp32.  The fp32 MFMA and the VALU have the same published peak,
// and without packed fp32 math the VALU reaches only half of it, so the matrix
// core is the only way to the fp32 roofline here.
//
// LDS layouts (64 four-byte banks; a wave's 64 single-float fragment reads
// must touch 64 distinct banks).  Both tiles keep their global layout:
//   * A as As[m][k], rows of 32 floats padded to 34: lane (m, h) reads
//     As[m][2 s + h]; the bank is (34 m + 2 s + h) mod 64, and 34 m mod 64 is
//     2 m for even m and 2 m + 32 for odd m, so the 64 lanes hit 64 banks.
//     A row segment is written as two 8-byte stores (rows are 8-byte aligned);
//   * B as Bs[k][n], rows of 128 floats padded to 160: lanes h = 0 and h = 1
//     read rows 2 s and 2 s + 1, 160 floats = 32 banks apart, so the two
//     halves of the wave cover disjoint banks; rows are written with 16-byte
//     stores.
// Out-of-range rows and columns are zero-filled on load and never stored
// (the edge handling of section 10.6 of the same page).
//
// The MFMAs take the B fragment as their first operand and the A fragment as
// their second, so each 32 x 32 block holds the transposed product: register
// r of lane l is C[row l % 32][column 8 (r / 4) + 4 (l / 32) + r % 4], and
// the epilogue reads and writes C in 16-byte pieces.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kLdA = kBK + 2;   // floats per As row (one m)
constexpr int kLdB = kBN + 32;  // floats per Bs row (one k)
constexpr int kThreads = 256;
constexpr int kAChunks = kBM * kBK / 4 / kThreads;  // float4 chunks of A per thread (4)
constexpr int kBChunks = kBK * kBN / 4 / kThreads;  // float4 chunks of B per thread (4)

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float *__restrict__ base, size_t row_off, int col,
                                       int ncols, bool row_ok) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
        // ncols % 4 == 0 and col % 4 == 0: the chunk is wholly in or out
        if (row_ok && col < ncols) v = *reinterpret_cast<const f32x4 *>(base + row_off + col);
    } else if (row_ok) {
        if (col + 0 < ncols) v.x = base[row_off + col + 0];
        if (col + 1 < ncols) v.y = base[row_off + col + 1];
        if (col + 2 < ncols) v.z = base[row_off + col + 2];
        if (col + 3 < ncols) v.w = base[row_off + col + 3];
    }
    return v;
}

template <bool VEC, bool EPI>
__global__ __launch_bounds__(kThreads, 2) void f32_mfma_kernel(int M, int N, int K, float alpha,
                                                               float beta,
                                                               const float *__restrict__ A,
                                                               const float *__restrict__ B,
                                                               float *C, int tiles_m,
                                                               int tiles_n, Epi epi) {
    __shared__ __attribute__((aligned(16))) float As[2][kBM][kLdA];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBK][kLdB];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // Global -> register staging.  A chunk c: row c / 8, k-quad c % 8 (eight
    // lanes cover one 128-byte row segment).  B chunk c: k-row c / 32,
    // n-quad c % 32 (a wave covers two 512-byte row segments).
    f32x4 ra[kAChunks], rb[kBChunks];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + kThreads * i;
            const int row = m0 + (c >> 3);
            ra[i] = load4<VEC>(A, static_cast<size_t>(row) * K, k0 + (c & 7) * 4, K, row < M);
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int c = tid + kThreads * i;
            const int kr = k0 + (c >> 5);
            rb[i] = load4<VEC>(B, static_cast<size_t>(kr) * N, n0 + (c & 31) * 4, N, kr < K);
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + kThreads * i;
            const int r = c >> 3, kq = (c & 7) * 4;
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<f32x2 *>(&As[buf][r][kq]) = f32x2{ra[i].x, ra[i].y};
            *reinterpret_cast<f32x2 *>(&As[buf][r][kq + 2]) = f32x2{ra[i].z, ra[i].w};
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<f32x4 *>(&Bs[buf][c >> 5][(c & 31) * 4]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int ktiles = (K + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ktiles) load_tile((t + 1) * kBK);
        // Fragments are double-buffered in registers: the reads of k-pair
        // s + 1 are issued before the four MFMAs of pair s, so the LDS
        // latency hides behind 256 cycles of matrix work (the scheduling
        // barriers keep the compiler from sinking the reads back).
        float fa[2][2], fb[2][2];
        auto read_frags = [&](int s, int buf) {
            const int kk = 2 * s + h;
            fa[buf][0] = As[cur][wm * 64 + l32][kk];
            fa[buf][1] = As[cur][wm * 64 + 32 + l32][kk];
            fb[buf][0] = Bs[cur][kk][wn * 64 + l32];
            fb[buf][1] = Bs[cur][kk][wn * 64 + 32 + l32];
        };
        read_frags(0, 0);
#pragma unroll
        for (int s = 0; s < kBK / 2; ++s) {
            const int buf = s & 1;
            if (s + 1 < kBK / 2) read_frags(s + 1, buf ^ 1);
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][0], fa[buf][0], acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][1], fa[buf][0], acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][0], fa[buf][1], acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][1], fa[buf][1], acc[1][1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t + 1 < ktiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: block (i, j) register 4 g + e of lane l is C[row][col + e]
    // with row = wm 64 + 32 i + l % 32 and col = wn 64 + 32 j + 8 g + 4 (l / 32).
    // With VEC (N % 4 == 0) a 4-column group is wholly inside or outside C
    // and C rows are 16-byte aligned when C is, which the caller checked.
    // With VEC and beta != 0 every C load is issued before the first store
    // (a load the compiler placed after a store to C would wait for it).
    f32x4 cin[2][2][4];
    // the fused epilogue's bias, by (j, g): the same columns for both i, and
    // loaded before any store for the same reason as C
    f32x4 bvs[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            bvs[j][g] = bias4<EPI>(epi.bias, n0 + wn * 64 + 32 * j + 8 * g + 4 * h, N);
    if (VEC && beta != 0.0f) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = m0 + wm * 64 + 32 * i + l32;
                    const int col = n0 + wn * 64 + 32 * j + 8 * g + 4 * h;
                    cin[i][j][g] =
                        (row < M && col < N)
                            ? *reinterpret_cast<const f32x4 *>(C + static_cast<size_t>(row) * N + col)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
                }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = m0 + wm * 64 + 32 * i + l32;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * 64 + 32 * j + 8 * g + 4 * h;
                if (row >= M) continue;
                float *c = C + static_cast<size_t>(row) * N + col;
                const f32x4 bv = bvs[j][g];
                if (VEC) {
                    if (col >= N) continue;
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = alpha * acc[i][j][4 * g + e];
                    if (beta != 0.0f) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, cin[i][j][g][e], out[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = epi_apply<EPI>(out[e], bv[e], epi.act);
                    *reinterpret_cast<f32x4 *>(c) = out;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (col + e < N) {
                            float out = alpha * acc[i][j][4 * g + e];
                            if (beta != 0.0f) out = fmaf(beta, c[e], out);
                            c[e] = epi_apply<EPI>(out, bv[e], epi.act);
                        }
                    }
                }
            }
        }
}

// ---- direct-to-LDS kernel (16-byte aligned rows, K < 2^21, N < 2^22) -------
// The same tiles, waves and MFMAs as f32_mfma_kernel, but:
//   * the next K tile goes global -> LDS with direct copies (lds_dma16: no
//     staging registers, no LDS write instructions, no wait until the end of
//     the step), issued at the start of the step into the other stage;
//   * MFMA k-pair s takes k = s from lanes 0-31 and k = 16 + s from lanes
//     32-63 (any pairing of the 32 k of a step sums the same products).  A
//     lane's A values for four consecutive pairs are then one 16-byte chunk,
//     read once for four pairs;
//   * MFMA block j's column c is C column wn 64 + 2 c + j, so a lane reads
//     its two blocks' B values for a pair as one 8-byte load, and the
//     epilogue interleaves the two blocks back into 8 consecutive columns.
// A direct copy writes 1 KB of LDS contiguously, so the padded layouts above
// are replaced by XOR swizzles of 16-byte chunks:
//   * A stage: 128 rows of 32 floats, chunk c of row m at position
//     c ^ ((m / 2) % 8): the 16 lanes served together by a 16-byte read fall
//     on 16 distinct bank groups;
//   * B stage: 32 rows of 128 floats, chunk c of row k at c ^ 8 ((k / 16) % 2):
//     the two lane halves of a read (rows s and 16 + s) sit 32 banks apart.
// Measured at 4096^3 against the register-staged kernel (1108-1116 us):
// direct copies 1064-1070 us, plus the permuted k pairs 1012 us, plus the
// B swizzle on k / 16 993-1000 us, plus the paired B reads 989 us (139
// TFLOP/s).  Spreading the copies over the step gained nothing.
// Rows past M, B rows past K, and chunks past K (A) or N (B) read zeros.
__device__ __forceinline__ int swz_fa(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int swz_fb(int k) { return ((k >> 4) & 1) << 3; }

template <bool EPI>
__global__ __launch_bounds__(kThreads, 2) void f32_dma_kernel(int M, int N, int K, float alpha,
                                                             float beta,
                                                             const float *__restrict__ A,
                                                             const float *__restrict__ B,
                                                             float *C, int tiles_m, int tiles_n,
                                                             Epi epi) {
    __shared__ __attribute__((aligned(16))) float As[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBK * kBN];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // copies: A wave-load L = 4 q + wave covers rows 8 L .. 8 L + 7 (lane p:
    // row 8 L + p / 8, position p % 8); B wave-load L covers rows 2 L, 2 L + 1
    // (lane p: row 2 L + p / 32, position p % 32).
    const int a_row = 8 * wave + (lane >> 3);             // + 32 q
    const int a_lc = (lane & 7) ^ swz_fa(a_row);          // swz_fa(a_row + 32 q) = swz_fa(a_row)
    const int b_row = 2 * wave + (lane >> 5);             // + 8 q
    // rows b_row + 8 q: swz_fb = 8 (q / 2) since b_row < 8
    auto b_lc = [&](int q) { return (lane & 31) ^ ((q >> 1) << 3); };
    auto issue_tile = [&](int k0, int buf) {
        const i32x4 ra = make_desc(A + static_cast<size_t>(m0) * K, static_cast<long long>(M - m0) * K * 4);
        const i32x4 rb = make_desc(B + static_cast<size_t>(k0) * N + n0,
                                  (static_cast<long long>(K - k0) * N - n0) * 4);
        const bool a_k_ok = k0 + 4 * a_lc < K;
        const uint32_t la = lds_address(&As[buf][0]), lb = lds_address(&Bs[buf][0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = a_row + 32 * q;
            const uint32_t off = a_k_ok ? static_cast<uint32_t>((row * K + k0 + 4 * a_lc) * 4) : kOOB;
            lds_dma16(ra, la + (4 * q + wave) * 1024, off);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = b_row + 8 * q;
            const int lc = b_lc(q);
            const uint32_t off = (n0 + 4 * lc < N) ? static_cast<uint32_t>((row * N + 4 * lc) * 4) : kOOB;
            lds_dma16(rb, lb + (4 * q + wave) * 1024, off);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int ktiles = (K + kBK - 1) / kBK;
    issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ktiles) issue_tile((t + 1) * kBK, cur ^ 1);
        // k-pair s of the MFMAs takes k = s from lanes 0-31 and k = 16 + s
        // from lanes 32-63 (any pairing of the 32 k sums the same products),
        // so a lane's A values for four consecutive pairs are one 16-byte
        // chunk: one read for four pairs.
        f32x4 fa4[2];
        float fb[2][2];
        auto read_a = [&](int u) {  // pairs 4u .. 4u + 3
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = wm * 64 + 32 * i + l32;
                fa4[i] = *reinterpret_cast<const f32x4 *>(
                    &As[cur][m * kBK + (((4 * h + u) ^ swz_fa(m)) << 2)]);
            }
        };
        // B: MFMA block j's column c is C column wn 64 + 2 c + j, so a lane
        // reads its two blocks' B values as one 8-byte pair.
        auto read_b = [&](int s, int buf) {
            const int kk = 16 * h + s;
            const int n = wn * 64 + 2 * l32;
            typedef float f32x2v __attribute__((ext_vector_type(2)));
            const f32x2v v = *reinterpret_cast<const f32x2v *>(
                &Bs[cur][kk * kBN + (((n >> 2) ^ swz_fb(kk)) << 2) + (n & 3)]);
            fb[buf][0] = v.x;
            fb[buf][1] = v.y;
        };
        f32x4 fa_cur[2];
        read_a(0);
        read_b(0, 0);
#pragma unroll
        for (int s = 0; s < kBK / 2; ++s) {
            const int buf = s & 1;
            if ((s & 3) == 0) {
                fa_cur[0] = fa4[0];
                fa_cur[1] = fa4[1];
                if (s + 4 < kBK / 2) read_a((s >> 2) + 1);
            }
            if (s + 1 < kBK / 2) read_b(s + 1, buf ^ 1);
            const float a0 = fa_cur[0][s & 3], a1 = fa_cur[1][s & 3];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][0], a0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][1], a0, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][0], a1, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[buf][1], a1, acc[1][1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // own copies of tile t+1 landed, own reads done
        __syncthreads();
    }

    // Epilogue: register 4 g + e of block (i, j) of lane l is C[row][col]
    // with row = wm 64 + 32 i + l % 32 and col = wn 64 + 16 g + 8 (l / 32) +
    // 2 e + j: the two blocks interleave into 8 consecutive columns.  With
    // beta != 0 every C load is issued before the first store: the compiler
    // cannot tell the loads from the stores to C apart, so a load placed
    // after a store would wait for it (one memory round trip per store).
    f32x4 cin[2][4][2];
    // the fused epilogue's bias, by (g, half), loaded before any store
    f32x4 bvs[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int half = 0; half < 2; ++half)
            bvs[g][half] = bias4<EPI>(epi.bias, n0 + wn * 64 + 16 * g + 8 * h + 4 * half, N);
    if (beta != 0.0f) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int row = m0 + wm * 64 + 32 * i + l32;
                    const int col = n0 + wn * 64 + 16 * g + 8 * h + 4 * half;
                    cin[i][g][half] =
                        (row < M && col < N)
                            ? *reinterpret_cast<const f32x4 *>(C + static_cast<size_t>(row) * N + col)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
                }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + wm * 64 + 32 * i + l32;
        if (row >= M) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int col = n0 + wn * 64 + 16 * g + 8 * h + 4 * half;
                if (col >= N) continue;
                float *c = C + static_cast<size_t>(row) * N + col;
                f32x4 out;
                out[0] = alpha * acc[i][0][4 * g + 2 * half];
                out[1] = alpha * acc[i][1][4 * g + 2 * half];
                out[2] = alpha * acc[i][0][4 * g + 2 * half + 1];
                out[3] = alpha * acc[i][1][4 * g + 2 * half + 1];
                if (beta != 0.0f) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = fmaf(beta, cin[i][g][half][e], out[e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = epi_apply<EPI>(out[e], bvs[g][half][e], epi.act);
                *reinterpret_cast<f32x4 *>(c) = out;
            }
        }
    }
}

}  // namespace

const char *f32_mfma_name(bool vec) {
    return vec ? "f32_mfma_128x128x32_vec4" : "f32_mfma_128x128x32_scalar";
}

template <bool EPI>
hipError_t launch_f32(int M, int N, int K, float alpha, float beta, const float *A,
                      const float *B, float *C, bool vec, const Epi &epi, hipStream_t stream) {
    const long long tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tiles)), block(kThreads);
    const int tm = static_cast<int>(tiles_m), tn = static_cast<int>(tiles_n);
    if (vec && K < (1 << 21) && N < (1 << 22))
        f32_dma_kernel<EPI><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C, tm, tn,
                                                        epi);
    else if (vec)
        f32_mfma_kernel<true, EPI><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                               tm, tn, epi);
    else
        f32_mfma_kernel<false, EPI><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                                tm, tn, epi);
    return hipGetLastError();
}

hipError_t launch_f32_mfma(int M, int N, int K, float alpha, float beta, const float *A,
                           const float *B, float *C, bool vec, const Epi &epi,
                           hipStream_t stream) {
    return epi_on(epi) ? launch_f32<true>(M, N, K, alpha, beta, A, B, C, vec, epi, stream)
                       : launch_f32<false>(M, N, K, alpha, beta, A, B, C, vec, epi, stream);
}

}  // namespace mgemm
