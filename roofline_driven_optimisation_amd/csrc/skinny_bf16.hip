// Decode-shaped bf16 GEMM (M <= 16): stream B from HBM exactly once.
//
// At M = 1..16 the arithmetic intensity is about M FLOP per byte, far left of
// the ridge, so the kernel is bound by HBM bandwidth (page "Memory hierarchy
// and cost table", section 4.6, small-batch GEMM row of the table) and follows
// the memory-bound checklist of page "Where kernel performance comes from":
// move every byte of B once, with coalesced 16-byte loads, and keep enough
// loads in flight.
//
// Work split.  A workgroup (4 waves) owns 128 output columns and a slice of
// K; the slices of one column block are `splits` workgroups, so the grid has
// (N / 128) * splits workgroups and fills all 256 CUs even when N = 4096.
// Inside a workgroup the waves take turns over 32-row k-blocks, two at a
// time, so each lane has sixteen 16-byte loads in flight.
//
// Per k-block, lane l loads eight B rows (k = 32 kb + 8 (l / 16) + e) at
// columns 8 (l % 16) .. +7: sixteen lanes read 256 contiguous bytes of a row.
// The 8 x 8 block is transposed in registers into eight k-octets, one per
// column, which are the B operands of eight v_mfma_f32_16x16x32_bf16; the A
// operand (row l % 16 of A, k-octet l / 16) is zero for rows >= M.  MFMA
// turns the M * 8 multiply-adds per loaded 16 bytes into a few instructions,
// where fp32 VALU work would not keep up with HBM at M = 16.
//
// Reduction.  The four waves' accumulators are summed through LDS.  With one
// split the workgroup applies alpha/beta and writes C.  Otherwise it writes
// its partial sums to a workspace, and the last workgroup of the column
// block to finish (found with an atomic counter; the pages do not cover this
// step) adds the partials in split order 0, 1, 2, ..., so results do not
// depend on timing, applies alpha/beta, writes C and re-arms the counter.
//
// Cross-XCD visibility.  The eight XCDs of an MI355X have private L2 caches.
// A device-scope fence makes a workgroup's stores visible to the others by
// writing back and invalidating its whole L2, which measured 3-10x slower
// than the streaming itself when every split workgroup does it.  The
// workspace (partials and counters) is therefore allocated uncached
// (hipDeviceMallocUncached): its loads and stores bypass the L2s and reach
// memory directly.  A writer waits until its partial stores are acknowledged
// (s_waitcnt 0) before the barrier and the counter increment, and the last
// workgroup reads the partials only after its atomic has returned, so it
// observes every partial without any L2 maintenance.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKBlock = 32;  // k rows per MFMA step
constexpr int kUnroll = 2;   // k-blocks in flight per wave

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(kThreads) void skinny_kernel(int M, int N, int K, float alpha,
                                                          float beta,
                                                          const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B,
                                                          float *C, int splits, int kblk_per_split,
                                                          float *partials, int *counters) {
    __shared__ f32x4 red[kWaves][8][64];
    __shared__ int s_last;

    const int cb = blockIdx.x / splits;
    const int sp = blockIdx.x - cb * splits;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4;      // k-octet inside a 32-row k-block
    const int cg = lane & 15;     // 8-column group inside the 128-column block
    const int n = cb * kSkinnyCols + cg * 8;
    const bool n_ok = n < N;
    const int m_a = lane & 15;    // row of A this lane feeds to the MFMA
    const bool m_ok = m_a < M;

    const int total_kblk = (K + kKBlock - 1) / kKBlock;
    const int kb_begin = sp * kblk_per_split;
    const int kb_end = min(kb_begin + kblk_per_split, total_kblk);

    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = kb_begin + wave; kb < kb_end; kb += kWaves * kUnroll) {
        u32x4 rb[kUnroll][8];
        u32x4 ra[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kbu = kb + u * kWaves;
            const bool blk_ok = kbu < kb_end;
            const int k0 = kbu * kKBlock + q * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (blk_ok && n_ok && k0 + e < K)
                    v = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(B + static_cast<size_t>(k0 + e) * N + n));
                rb[u][e] = v;
            }
            u32x4 a = {0u, 0u, 0u, 0u};
            if (blk_ok && m_ok && k0 < K)
                a = *reinterpret_cast<const u32x4 *>(A + static_cast<size_t>(m_a) * K + k0);
            ra[u] = a;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bf16x8 a = as_bf16x8(ra[u]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                // column t of the 8 x 8 block as eight k-consecutive bf16
                const int d = t >> 1;
                u32x4 col;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    col[w] = (t & 1) ? pack_hi(rb[u][2 * w][d], rb[u][2 * w + 1][d])
                                     : pack_lo(rb[u][2 * w][d], rb[u][2 * w + 1][d]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(col), acc[t], 0, 0, 0);
            }
        }
    }

    // acc[t] register r of lane l is row 4 (l / 16) + r, column 8 (l % 16) + t
    // of the block.  Sum the four waves through LDS.
#pragma unroll
    for (int t = 0; t < 8; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();

    const int l = tid & 63, r = tid >> 6;
    const int m = 4 * (l >> 4) + r;
    const int nn = cb * kSkinnyCols + 8 * (l & 15);
    const bool ok = m < M && nn < N;
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += red[w][t][l][r];
        v[t] = s;
    }

    if (splits == 1) {
        if (ok) {
            float *c = C + static_cast<size_t>(m) * N + nn;
            f32x4 o0, o1;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o0[t] = alpha * v[t];
                o1[t] = alpha * v[t + 4];
            }
            if (beta != 0.0f) {
                const f32x4 c0 = reinterpret_cast<const f32x4 *>(c)[0];
                const f32x4 c1 = reinterpret_cast<const f32x4 *>(c)[1];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    o0[t] = fmaf(beta, c0[t], o0[t]);
                    o1[t] = fmaf(beta, c1[t], o1[t]);
                }
            }
            reinterpret_cast<f32x4 *>(c)[0] = o0;
            reinterpret_cast<f32x4 *>(c)[1] = o1;
        }
        return;
    }

    if (ok) {
        f32x4 *p = reinterpret_cast<f32x4 *>(partials + (static_cast<size_t>(sp) * M + m) * N + nn);
        p[0] = f32x4{v[0], v[1], v[2], v[3]};
        p[1] = f32x4{v[4], v[5], v[6], v[7]};
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&counters[cb], 1) == splits - 1);
    __syncthreads();
    if (!s_last) return;

    if (ok) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            const f32x4 *p =
                reinterpret_cast<const f32x4 *>(partials + (static_cast<size_t>(s) * M + m) * N + nn);
            s0 += p[0];
            s1 += p[1];
        }
        float *c = C + static_cast<size_t>(m) * N + nn;
        f32x4 o0 = alpha * s0, o1 = alpha * s1;
        if (beta != 0.0f) {
            const f32x4 c0 = reinterpret_cast<const f32x4 *>(c)[0];
            const f32x4 c1 = reinterpret_cast<const f32x4 *>(c)[1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o0[t] = fmaf(beta, c0[t], o0[t]);
                o1[t] = fmaf(beta, c1[t], o1[t]);
            }
        }
        reinterpret_cast<f32x4 *>(c)[0] = o0;
        reinterpret_cast<f32x4 *>(c)[1] = o1;
    }
    if (tid == 0) atomicExch(&counters[cb], 0);  // re-arm for the next call
}

}  // namespace

int skinny_pick_splits(int M, int N, int K, int num_cus) {
    (void)M;
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    const int target = num_cus + num_cus / 4;  // about 1.25 workgroups per CU (measured best)
    int splits = (target + col_blocks - 1) / col_blocks;
    const int max_splits = kblks / 8 > 1 ? kblks / 8 : 1;  // >= 8 k-blocks per workgroup
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    return splits;
}

hipError_t launch_skinny_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                              const uint16_t *B, float *C, int splits, float *partials,
                              int *counters, hipStream_t stream) {
    if (M < 1 || M > kSkinnyMaxM || splits < 1) return hipErrorInvalidValue;
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    int per = (kblks + splits - 1) / splits;
    if (per < 1) per = 1;
    // recompute so that no split is empty: each one must arrive at the counter
    const int real_splits = (kblks + per - 1) / per > 0 ? (kblks + per - 1) / per : 1;
    if (real_splits > 1 && (partials == nullptr || counters == nullptr)) return hipErrorInvalidValue;
    const long long grid = static_cast<long long>(col_blocks) * real_splits;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    skinny_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream>>>(
        M, N, K, alpha, beta, A, B, C, real_splits, per, partials, counters);
    return hipGetLastError();
}

}  // namespace mgemm
