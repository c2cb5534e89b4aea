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
// (N / 128) * splits workgroups.  One CU alone cannot keep enough loads in
// flight to draw more than a few tens of GB/s, so the grid is sized to a few
// workgroups per CU over all 256 CUs.  Inside a workgroup the waves take
// turns over 32-row k-blocks.  The loop is software-pipelined one k-block
// deep: the eight 16-byte B loads (and the A load) of a wave's next k-block
// are issued before its current k-block is multiplied, so every lane keeps
// 8 to 16 loads in flight the whole time, not just between compute bursts.
// At that depth a wave needs few enough registers for three workgroups per
// CU, which keeps more loads in flight per CU than a deeper pipeline at two.
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
// than the streaming itself when every split workgroup does it.  Two ways
// round it:
//   * uncached scratch (hipDeviceMallocUncached): partials and counters
//     bypass the L2s and reach memory directly.  A writer waits until its
//     partial stores are acknowledged (s_waitcnt 0) before the barrier and
//     the counter increment, and the last workgroup reads the partials only
//     after its atomic has returned, so it observes every partial without
//     any L2 maintenance;
//   * XCD-local placement: the hardware deals workgroups to the eight XCDs
//     in round-robin order, so workgroups whose ids are equal modulo 8 run on
//     one XCD (which XCD takes workgroup 0 varies from launch to launch; the
//     library checks the property once per device by reading the XCC_ID
//     hardware register from a probe grid).  So the splits of a column block
//     can all be put on one XCD.  Their partials and counter live in ordinary cached
//     memory that no other XCD touches; L2 is the point of coherence for
//     every CU of the XCD, so the same store / wait / atomic / load sequence
//     is correct, with each step an L2 round trip instead of a memory one.
//     Vector L1 caches are write-through and no line of a block's partials
//     is read before its last workgroup reads it, so no L1 holds a stale copy.
// Which column blocks share an XCD also decides which HBM channels the XCD
// streams from at once: runs of three adjacent blocks (768 bytes of each B
// row) measured faster than one, two, four or all of an XCD's blocks.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKBlock = 32;  // k rows per MFMA step
constexpr int kDepth = 1;    // k-blocks per pipeline stage
constexpr int kNonTemporal = 2;         // buffer-load cache policy: streaming (nt)
constexpr int kCounterLine = 32;        // ints per 128-byte line

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, long long bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

// The loads of one pipeline stage: kDepth k-blocks, each 8 B rows and one
// A octet per lane.
struct Stage {
    u32x4 b[kDepth][8];
    u32x4 a[kDepth];
};

// XCD_LOCAL selects the placement and scratch of the split-K reduction.
// false: workgroup b is split b / col_blocks of column block b % col_blocks
// (consecutive workgroups, dealt to the XCDs in turn, take adjacent column
// blocks: each XCD streams from all of B, which measured 4-7 % faster than
// giving the splits of a block consecutive ids); the partials of split s are
// the M x N matrix at partials + s M N and the counter of block cb is at
// counters + cb * counter_stride, all in uncached memory.
// true: with col_blocks = 8 q + r, the r trailing column blocks take the
// first r * splits workgroups (rounded up to a multiple of 8 by idle ones) and
// reduce as above.  Then the workgroups with b % 8 == x, which share one
// XCD, form group x, and j = b / 8
// (counted from the end of that first part) is split j % splits of the
// (j / splits)-th of the q column blocks given to XCD x: runs of xcd_group
// adjacent blocks, dealt to the groups in turn.  Group x uses only the
// scratch block at xcd_base + x * xcd_block_bytes (counters first, then the
// partials of its column blocks, 128 columns wide), so that part of the
// reduction stays in one XCD's L2.  Every XCD gets the same number of
// workgroups.  With all_local, r = 0 and q = ceil(col_blocks / 8): the
// placement is the same, and a workgroup whose block number comes out at or
// past col_blocks (the padding of the last round) exits at once.
template <bool XCD_LOCAL, bool EPI>
__global__ __launch_bounds__(kThreads) void skinny_kernel(int M, int N, int K, float alpha,
                                                          float beta,
                                                          const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B,
                                                          float *C, int splits, int kblk_per_split,
                                                          float *partials, int *counters,
                                                          int counter_stride, char *xcd_base,
                                                          long long xcd_block_bytes, int xcd_group,
                                                          int all_local, Epi epi) {
    __shared__ f32x4 red[kWaves][8][64];
    __shared__ int s_last;

    int cb, sp, cb_local = 0;
    bool local = false;  // uniform over the workgroup
    if (XCD_LOCAL) {
        const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
        // all_local: every column block is XCD-local, the last round of
        // blocks padded with idle workgroups; otherwise col_blocks % 8
        // blocks reduce through uncached memory
        const int rest = all_local ? 0 : col_blocks % kXcdCount;
        const int rest_groups = (rest * splits + kXcdCount - 1) / kXcdCount * kXcdCount;
        const int b = blockIdx.x;
        if (b < rest_groups) {
            if (b >= rest * splits) return;  // padding: exits before any barrier
            sp = b / rest;
            cb = col_blocks - rest + (b - sp * rest);
        } else {
            // rest_groups % 8 == 0, so (b - rest_groups) % 8 == b % 8
            const int x = b % kXcdCount, j = (b - rest_groups) / kXcdCount;
            local = true;
            cb_local = j / splits;
            sp = j - cb_local * splits;
            {
                const int q = all_local ? (col_blocks + kXcdCount - 1) / kXcdCount
                                        : col_blocks / kXcdCount;
                const int g = xcd_group;
                const int full = (q / g) * g;
                if (cb_local < full)
                    cb = (cb_local / g) * kXcdCount * g + x * g + cb_local % g;
                else
                    cb = full * kXcdCount + x * (q - full) + (cb_local - full);
            }
            if (cb >= col_blocks) return;  // all_local padding: exits before any barrier
            char *blk = xcd_base + static_cast<size_t>(x) * xcd_block_bytes;
            counters = reinterpret_cast<int *>(blk);
            counter_stride = kCounterLine;
            partials = reinterpret_cast<float *>(blk + kSkinnyXcdCounterInts * sizeof(int));
        }
    } else {
        const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
        sp = blockIdx.x / col_blocks;
        cb = blockIdx.x - sp * col_blocks;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4;      // k-octet inside a 32-row k-block
    const int cg = lane & 15;     // 8-column group inside the 128-column block
    const int m_a = lane & 15;    // row of A this lane feeds to the MFMA

    const int total_kblk = (K + kKBlock - 1) / kKBlock;
    const int kb_begin = sp * kblk_per_split;
    const int kb_end = min(kb_begin + kblk_per_split, total_kblk);
    // k-blocks of this wave: kb_begin + wave + 4 j, j = 0 .. nj - 1
    const int nj = max(0, (kb_end - kb_begin - wave + kWaves - 1) / kWaves);
    const int stages = (nj + kDepth - 1) / kDepth;

    // Buffer descriptors based at the slice origin (row kb_begin * 32 of B,
    // column cb * 128; column kb_begin * 32 of A), so that every offset used
    // fits in 32 bits.  Rows past the slice or past K, columns past N and
    // rows of A past M are given the out-of-range offset and read as zeros.
    const long long k_first = static_cast<long long>(kb_begin) * kKBlock;
    const __amdgpu_buffer_rsrc_t rb = rsrc(
        B + k_first * N + static_cast<long long>(cb) * kSkinnyCols,
        ((K - k_first) * N - static_cast<long long>(cb) * kSkinnyCols) * 2);
    const __amdgpu_buffer_rsrc_t ra =
        rsrc(A + k_first, (static_cast<long long>(M) * K - k_first) * 2);
    const int k_slice = (kb_end - kb_begin) * kKBlock;  // rows of B in this slice (<= K - k_first)
    const bool n_ok = cb * kSkinnyCols + cg * 8 < N;
    const bool m_ok = m_a < M;
    // row r (within the slice) of lane's B column group; k of A for this lane
    auto b_off = [&](int r) -> uint32_t {
        return (n_ok && r < k_slice && r + static_cast<int>(k_first) < K)
                   ? static_cast<uint32_t>((r * N + cg * 8) * 2) : kOOB;
    };
    auto a_off = [&](int kk) -> uint32_t {
        return (m_ok && kk < k_slice && kk + static_cast<int>(k_first) < K)
                   ? static_cast<uint32_t>((m_a * K + kk) * 2) : kOOB;
    };

    auto load_stage = [&](int st, Stage &x) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int j = st * kDepth + d;
            const int r0 = (j < nj) ? (wave + kWaves * j) * kKBlock + q * 8 : k_slice;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x.b[d][e] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, static_cast<int>(b_off(r0 + e)),
                                                                 0, kNonTemporal));
            x.a[d] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, static_cast<int>(a_off(r0)), 0, 0));
        }
    };

    // The fused epilogue's bias of the block's 128 columns, one per thread,
    // requested before the stream (one register over the loop) and parked
    // in LDS for the final store.
    __shared__ float s_bias[kSkinnyCols];
    float bias_mine = 0.0f;
    if constexpr (EPI) {
        const int nb = cb * kSkinnyCols + tid;
        if (epi.bias != nullptr && tid < kSkinnyCols && nb < N) bias_mine = epi.bias[nb];
    }

    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_stage = [&](const Stage &x) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const bf16x8 a = as_bf16x8(x.a[d]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                // column t of the 8 x 8 block as eight k-consecutive bf16
                const int w2 = t >> 1;
                u32x4 col;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    col[w] = (t & 1) ? pack_hi(x.b[d][2 * w][w2], x.b[d][2 * w + 1][w2])
                                     : pack_lo(x.b[d][2 * w][w2], x.b[d][2 * w + 1][w2]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(col), acc[t], 0, 0, 0);
            }
        }
    };

    // Two register stages: the loads of stage s+1 are in flight while stage
    // s is multiplied.
    Stage x0, x1;
    if (stages > 0) load_stage(0, x0);
    for (int st = 0; st < stages; st += 2) {
        if (st + 1 < stages) load_stage(st + 1, x1);
        compute_stage(x0);
        if (st + 1 < stages) {
            if (st + 2 < stages) load_stage(st + 2, x0);
            compute_stage(x1);
        }
    }

    // acc[t] register r of lane l is row 4 (l / 16) + r, column 8 (l % 16) + t
    // of the block.  Sum the four waves through LDS.
#pragma unroll
    for (int t = 0; t < 8; ++t) red[wave][t][lane] = acc[t];
    if (EPI && tid < kSkinnyCols) s_bias[tid] = bias_mine;
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

    auto store_c = [&](f32x4 o0, f32x4 o1) {
        float *c = C + static_cast<size_t>(m) * N + nn;
        if (beta != 0.0f) {
            const f32x4 c0 = reinterpret_cast<const f32x4 *>(c)[0];
            const f32x4 c1 = reinterpret_cast<const f32x4 *>(c)[1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o0[t] = fmaf(beta, c0[t], o0[t]);
                o1[t] = fmaf(beta, c1[t], o1[t]);
            }
        }
        if constexpr (EPI) {
            const int c0 = 8 * (l & 15);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o0[t] = epi_apply<EPI>(o0[t], s_bias[c0 + t], epi.act);
                o1[t] = epi_apply<EPI>(o1[t], s_bias[c0 + 4 + t], epi.act);
            }
        }
        reinterpret_cast<f32x4 *>(c)[0] = o0;
        reinterpret_cast<f32x4 *>(c)[1] = o1;
    };

    if (splits == 1) {
        if (ok)
            store_c(alpha * f32x4{v[0], v[1], v[2], v[3]}, alpha * f32x4{v[4], v[5], v[6], v[7]});
        return;
    }

    // one counter per column block, each on its own 128-byte line when the
    // counter block has room (atomics on one line are serialised)
    int *counter = counters + (local ? cb_local : cb) * counter_stride;
    // partials of split s for this lane: part + s * split_stride
    const float *part;
    size_t split_stride;
    if (local) {
        split_stride = static_cast<size_t>(M) * kSkinnyCols;
        part = partials + static_cast<size_t>(cb_local) * splits * split_stride +
               static_cast<size_t>(m) * kSkinnyCols + 8 * (l & 15);
    } else {
        split_stride = static_cast<size_t>(M) * N;
        part = partials + static_cast<size_t>(m) * N + nn;
    }
    if (ok) {
        f32x4 *p = reinterpret_cast<f32x4 *>(const_cast<float *>(part) + sp * split_stride);
        p[0] = f32x4{v[0], v[1], v[2], v[3]};
        p[1] = f32x4{v[4], v[5], v[6], v[7]};
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(counter, 1) == splits - 1);
    __syncthreads();
    if (!s_last) return;

    if (ok) {
        // Eight splits' partials are requested at a time and then added in
        // split order: one memory round trip per eight splits, and the same
        // summation order on every call.
        constexpr int kBatch = 8;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        for (int sb = 0; sb < splits; sb += kBatch) {
            f32x4 p0[kBatch], p1[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int s = min(sb + u, splits - 1);
                const f32x4 *p = reinterpret_cast<const f32x4 *>(part + s * split_stride);
                p0[u] = p[0];
                p1[u] = p[1];
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (sb + u < splits) {
                    s0 += p0[u];
                    s1 += p1[u];
                }
            }
        }
        store_c(alpha * s0, alpha * s1);
    }
    if (tid == 0) atomicExch(counter, 0);  // re-arm for the next call
}

}  // namespace

int skinny_pick_splits(int M, int N, int K, int num_cus, bool xcd_local) {
    // Measured on the decode shapes (4096 x 11008, 11008 x 4096, 4096 x
    // 32000, M = 1, 8, 16):
    //   * with about one 128-column block per CU already (the LM head: 250
    //     blocks) one split is best: every CU streams and no partials move
    //     (44.0 us against 47.4 us with eight splits);
    //   * otherwise, when the reduction stays in XCD-local L2, or at M <= 8,
    //     eight splits (688 or 256 workgroups): 21.5 us against 22.0 us with
    //     four at 16 x 4096 x 11008 with L2-local partials;
    //   * through uncached memory at M > 8, where the partials are 16x
    //     larger, the fewest splits that reach every CU, rounded up to a power
    //     of two, win (22.6 us with two splits against 24.0 us with eight at
    //     16 x 4096 x 11008);
    //   * at M <= 2 with few column blocks, sixteen XCD-local splits, when
    //     that is at most two workgroups per CU (1 x 11008 x 4096: 32 blocks,
    //     19.0 us against 19.4 us with eight; at M = 8 or 16 eight stay
    //     faster, their partials being larger).
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    const int need = (num_cus + col_blocks - 1) / col_blocks;
    int splits;
    if (10 * col_blocks >= 9 * num_cus) {
        splits = 1;
    } else if (xcd_local && M <= 2 && 16 * col_blocks <= 2 * num_cus) {
        splits = 16;
    } else if (M <= 8 || xcd_local) {
        splits = max(8, need);
    } else {
        splits = 2;
        while (splits < need) splits *= 2;
    }
    const int max_splits = kblks / 8 > 1 ? kblks / 8 : 1;  // >= 8 k-blocks per workgroup
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    return splits;
}

bool skinny_slice_fits(int M, int N, int K, int splits) {
    const int kblks = (K + kKBlock - 1) / kKBlock;
    if (splits < 1) splits = 1;
    const int per = (kblks + splits - 1) / splits > 0 ? (kblks + splits - 1) / splits : 1;
    return static_cast<long long>(per) * kKBlock * N * 2 < 0x7fff0000LL &&
           static_cast<long long>(M) * K * 2 < 0x7fff0000LL;
}

hipError_t launch_skinny_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                              const uint16_t *B, float *C, int splits, float *partials,
                              int *counters, int counter_ints, const Epi &epi,
                              hipStream_t stream) {
    if (M < 1 || M > kSkinnyMaxM || splits < 1) return hipErrorInvalidValue;
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    int per = (kblks + splits - 1) / splits;
    if (per < 1) per = 1;
    // 32-bit buffer offsets: one slice of B and all of A must stay below 2^31 bytes
    if (static_cast<long long>(per) * kKBlock * N * 2 >= 0x7fff0000LL ||
        static_cast<long long>(M) * K * 2 >= 0x7fff0000LL)
        return hipErrorInvalidValue;
    // recompute so that no split is empty: each one must arrive at the counter
    const int real_splits = (kblks + per - 1) / per > 0 ? (kblks + per - 1) / per : 1;
    if (real_splits > 1 && (partials == nullptr || counters == nullptr)) return hipErrorInvalidValue;
    const long long grid = static_cast<long long>(col_blocks) * real_splits;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int counter_stride = col_blocks * kCounterLine <= counter_ints ? kCounterLine : 1;
    if (real_splits > 1 && col_blocks > counter_ints) return hipErrorInvalidValue;
    const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
    if (epi_on(epi))
        skinny_kernel<false, true><<<g, blk, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                          real_splits, per, partials, counters,
                                                          counter_stride, nullptr, 0, 1, 0, epi);
    else
        skinny_kernel<false, false><<<g, blk, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                           real_splits, per, partials, counters,
                                                           counter_stride, nullptr, 0, 1, 0, epi);
    return hipGetLastError();
}

namespace {

// Fills xcc[b] with the XCD that workgroup b ran on (hardware register
// XCC_ID, bits 3:0).  Its LDS footprint allows one workgroup per CU, so most
// of the grid is dispatched late, as earlier workgroups retire (their busy
// times differ, so they retire out of order).
__global__ __launch_bounds__(256) void xcd_probe_kernel(int *xcc, int count) {
    __shared__ float fill[36 * 1024];  // 144 KB
    const int id = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
    fill[threadIdx.x] = static_cast<float>(threadIdx.x);
    const long long t0 = clock64();
    const long long busy = 500LL * (1 + (blockIdx.x * 7919u) % 13);
    while (clock64() - t0 < busy) {
    }
    __syncthreads();
    if (threadIdx.x == 0 && static_cast<int>(blockIdx.x) < count)
        xcc[blockIdx.x] = id + static_cast<int>(fill[1]) * 0;
}

}  // namespace

hipError_t probe_xcd_mapping(bool *ok, hipStream_t stream, int *buffer) {
    *ok = false;
    constexpr int kProbeGroups = kXcdProbeInts;
    int *d = buffer;
    hipError_t e = hipSuccess;
    if (d == nullptr && (e = hipMalloc(&d, kProbeGroups * sizeof(int))) != hipSuccess) return e;
    static int h[kProbeGroups];
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    xcd_probe_kernel<<<dim3(kProbeGroups), dim3(256), 0, stream>>>(d, kProbeGroups);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(h, d, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (buffer == nullptr) (void)hipFree(d);
    if (e != hipSuccess) return e;
    // The XCD of workgroup 0 varies between launches (the dispatcher's
    // round robin can carry over from earlier work); what the kernels rely
    // on is that workgroups b and b' with b % 8 == b' % 8 share an XCD and
    // that the eight residues cover eight different XCDs.
    bool all = true;
    unsigned seen = 0;
    for (int b = 0; b < kXcdCount; ++b) {
        all = all && h[b] >= 0 && h[b] < 32 && !(seen & (1u << h[b]));
        if (h[b] >= 0 && h[b] < 32) seen |= 1u << h[b];
    }
    for (int b = kXcdCount; b < kProbeGroups; ++b) all = all && h[b] == h[b % kXcdCount];
    *ok = all;
    return hipSuccess;
}

bool skinny_xcd_local_fits(int M, int N, int K, int splits, size_t block_bytes, bool all_local) {
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    const int per = (kblks + splits - 1) / splits > 0 ? (kblks + splits - 1) / splits : 1;
    const int real_splits = (kblks + per - 1) / per;
    // XCD-local column blocks per XCD
    const int mine = all_local ? (col_blocks + kXcdCount - 1) / kXcdCount : col_blocks / kXcdCount;
    if (real_splits < 2 || M < 1 || M > kSkinnyMaxM || mine < 1) return false;
    if (mine * kCounterLine > kSkinnyXcdCounterInts) return false;
    const size_t head = kSkinnyXcdCounterInts * sizeof(int);
    return block_bytes > head &&
           static_cast<unsigned long long>(mine) * real_splits * M * kSkinnyCols * sizeof(float) <=
               block_bytes - head;
}

hipError_t launch_skinny_bf16_xcd(int M, int N, int K, float alpha, float beta,
                                  const uint16_t *A, const uint16_t *B, float *C, int splits,
                                  float *partials, int *counters, int counter_ints,
                                  char *xcd_base, size_t xcd_block_bytes, int xcd_group,
                                  bool all_local, const Epi &epi, hipStream_t stream) {
    if (xcd_base == nullptr ||
        !skinny_xcd_local_fits(M, N, K, splits, xcd_block_bytes, all_local))
        return hipErrorInvalidValue;
    const int col_blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
    const int kblks = (K + kKBlock - 1) / kKBlock;
    const int per = (kblks + splits - 1) / splits;
    if (static_cast<long long>(per) * kKBlock * N * 2 >= 0x7fff0000LL ||
        static_cast<long long>(M) * K * 2 >= 0x7fff0000LL)
        return hipErrorInvalidValue;
    const int real_splits = (kblks + per - 1) / per;
    const int rest = all_local ? 0 : col_blocks % kXcdCount;
    if (rest > 0 && (partials == nullptr || counters == nullptr || col_blocks > counter_ints))
        return hipErrorInvalidValue;
    const int counter_stride = col_blocks * kCounterLine <= counter_ints ? kCounterLine : 1;
    const long long rest_groups =
        (static_cast<long long>(rest) * real_splits + kXcdCount - 1) / kXcdCount * kXcdCount;
    const long long local_blocks =
        all_local ? static_cast<long long>((col_blocks + kXcdCount - 1) / kXcdCount) * kXcdCount
                  : col_blocks - rest;
    const long long grid = rest_groups + local_blocks * real_splits;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g(static_cast<unsigned>(grid)), blk(kThreads);
    const int grp = xcd_group < 1 ? 1 : xcd_group;
    const long long bb = static_cast<long long>(xcd_block_bytes);
    const int al = all_local ? 1 : 0;
    if (epi_on(epi))
        skinny_kernel<true, true><<<g, blk, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                         real_splits, per, partials, counters,
                                                         counter_stride, xcd_base, bb, grp, al,
                                                         epi);
    else
        skinny_kernel<true, false><<<g, blk, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                          real_splits, per, partials, counters,
                                                          counter_stride, xcd_base, bb, grp, al,
                                                          epi);
    return hipGetLastError();
}

}  // namespace mgemm
