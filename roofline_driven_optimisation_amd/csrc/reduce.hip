// Sum of a float32 vector: the memory-bound case study of page "Memory
// hierarchy and cost table", section 4.7, which sums 100 million floats and
// moves from one 4-byte load per thread with an LDS tree and a global atomic
// (45 % of HBM on its GPU) to 16-byte loads, register sums and one atomic per
// block (91 %).  Two kernels here:
//
// reduce_kernel (the optimised form, sized for MI355X):
//   * every workgroup owns one contiguous chunk of the 16-byte aligned body
//     and streams it with 16-byte non-temporal loads, eight in flight per
//     lane (a wave reads 1 KB per load, a workgroup 4 KB), the pattern that
//     measured 6.1-6.35 TB/s for a plain read on MI355X;
//   * a lane keeps four fp32 accumulators (one per element of its 16-byte
//     loads), adds them pairwise, and the workgroup sums its 256 lanes with
//     an LDS tree;
//   * there is no floating-point atomic (its order would vary from run to
//     run): each workgroup posts its partial to uncached scratch and the
//     last one to finish (an integer atomic counter) sums the partials with
//     a fixed tree, adds the up to six unaligned head and tail elements and
//     writes the result.  The result does not depend on timing.
//
// reduce_tree_kernel (the page's first version, kept as the ladder's first
// rung): one element per thread and an LDS tree per 256 elements, launched
// again on its own partials until one value is left (a tree in place of the
// page's atomic, so the result is deterministic too).
//
// Rounding: an element passes through at most chunk / (256 * 4) + 2 + 8 +
// 8 + 8 + 6 fp32 additions in reduce_kernel (its accumulator, the pairwise
// sums, the block tree, the 8-partial chain, the final tree, the unaligned
// ends), and ceil(log2 n) in reduce_tree_kernel.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kRedThreads = 256;
constexpr int kRedInFlight = 8;  // 16-byte loads per lane per iteration
constexpr int kNonTemporalLoad = 2;

__device__ __forceinline__ float block_tree_sum(float v, float *red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
#pragma unroll
    for (int s = kRedThreads / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    return red[0];
}

// body: 16-byte aligned, n4 groups of four floats; per_block groups per
// workgroup (the last one may have fewer).  The n_head elements before the
// body and the n_tail after it (at most 3 each) are added by the last
// workgroup, head first.
__device__ __forceinline__ float add_ends(float t, const float *head, int n_head,
                                          const float *tail, int n_tail) {
    for (int e = 0; e < n_head; ++e) t += head[e];
    for (int e = 0; e < n_tail; ++e) t += tail[e];
    return t;
}

__global__ __launch_bounds__(kRedThreads) void reduce_kernel(const float *body, long long n4,
                                                             long long per_block,
                                                             const float *head, int n_head,
                                                             const float *tail, int n_tail,
                                                             float *partials, int *counter,
                                                             float *out) {
    __shared__ float red[kRedThreads];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const long long first = static_cast<long long>(b) * per_block;
    long long count = n4 - first;
    if (count > per_block) count = per_block;
    if (count < 0) count = 0;
    // descriptor over this workgroup's chunk only (count * 16 < 2^31 bytes)
    const __amdgpu_buffer_rsrc_t r = make_rsrc(body + first * 4, count * 16);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int iters = static_cast<int>((count + kRedThreads * kRedInFlight - 1) /
                                       (kRedThreads * kRedInFlight));
    for (int it = 0; it < iters; ++it) {
        f32x4 v[kRedInFlight];
#pragma unroll
        for (int u = 0; u < kRedInFlight; ++u) {
            const long long g =
                (static_cast<long long>(it) * kRedInFlight + u) * kRedThreads + tid;
            const uint32_t off = g < count ? static_cast<uint32_t>(g * 16) : kOOB;
            v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, static_cast<int>(off), 0, kNonTemporalLoad));
        }
#pragma unroll
        for (int u = 0; u < kRedInFlight; ++u) acc += v[u];
    }
    const float mine = (acc.x + acc.y) + (acc.z + acc.w);
    const float block_sum = block_tree_sum(mine, red);

    if (gridDim.x == 1) {  // a single workgroup needs no second stage
        if (tid == 0) *out = add_ends(block_sum, head, n_head, tail, n_tail);
        return;
    }
    // Post the partial (uncached memory: it reaches the device's memory, so
    // the last workgroup sees it whatever XCD it runs on), wait for the
    // store to be acknowledged, then count this workgroup in.
    if (tid == 0) partials[b] = block_sum;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(counter, 1) == static_cast<int>(gridDim.x) - 1);
    __syncthreads();
    if (!s_last) return;
    // Last workgroup: lane t sums partials 8 t .. 8 t + 7 in order, then the
    // block tree; a fixed order, so the result does not depend on timing.
    float s = 0.0f;
    const int nb = static_cast<int>(gridDim.x);
    static_assert(kReduceMaxBlocks <= 8 * kRedThreads, "8 partials per lane");
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = tid * 8 + u;
        if (i < nb) s += __hip_atomic_load(partials + i, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
    }
    const float total = block_tree_sum(s, red);
    if (tid == 0) {
        *out = add_ends(total, head, n_head, tail, n_tail);
        atomicExch(counter, 0);  // re-arm for the next call
    }
}

// One element per thread, an LDS tree per 256 elements: out[b] = sum of
// in[256 b .. 256 b + 255].
__global__ __launch_bounds__(kRedThreads) void reduce_tree_kernel(const float *in, long long n,
                                                                  float *out) {
    __shared__ float red[kRedThreads];
    const long long i = static_cast<long long>(blockIdx.x) * kRedThreads + threadIdx.x;
    const float v = i < n ? in[i] : 0.0f;
    const float s = block_tree_sum(v, red);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

}  // namespace

long long reduce_blocks(long long n, int num_cus) {
    // a few workgroups per CU, each with a chunk of at least 64 KB
    const long long n4 = n / 4;
    // (16 per CU, 4096 in all, measured 77 us against 67 us at 10^8)
    long long blocks = static_cast<long long>(num_cus) * 8;
    const long long min_chunk4 = 4096;  // float4 groups
    if (n4 < blocks * min_chunk4) blocks = (n4 + min_chunk4 - 1) / min_chunk4;
    if (blocks < 1) blocks = 1;
    if (blocks > kReduceMaxBlocks) blocks = kReduceMaxBlocks;
    return blocks;
}

hipError_t launch_reduce_sum(const float *x, long long n, float *out, float *partials,
                             int *counter, int blocks, hipStream_t stream) {
    const uintptr_t addr = reinterpret_cast<uintptr_t>(x);
    if (n < 0 || (addr & 3) != 0 || blocks < 1 || blocks > kReduceMaxBlocks ||
        (blocks > 1 && (partials == nullptr || counter == nullptr)))
        return hipErrorInvalidValue;
    // unaligned head (up to the first 16-byte boundary), aligned body, tail
    long long head = static_cast<long long>(((16 - (addr & 15)) & 15) / 4);
    if (head > n) head = n;
    const long long n4 = (n - head) / 4;
    const long long tail = n - head - 4 * n4;
    const long long per_block = (n4 + blocks - 1) / blocks;
    if (per_block * 16 > 0x7fff0000LL) return hipErrorInvalidValue;
    reduce_kernel<<<dim3(blocks), dim3(kRedThreads), 0, stream>>>(
        x + head, n4, per_block > 0 ? per_block : 1, x, static_cast<int>(head),
        x + head + 4 * n4, static_cast<int>(tail), partials, counter, out);
    return hipGetLastError();
}

hipError_t launch_reduce_sum_tree(const float *x, long long n, float *out, float *scratch,
                                  long long scratch_floats, hipStream_t stream) {
    if (n < 0) return hipErrorInvalidValue;
    if (n == 0) {
        reduce_tree_kernel<<<dim3(1), dim3(kRedThreads), 0, stream>>>(x, 0, out);
        return hipGetLastError();
    }
    // level sizes shrink 256-fold; ping-pong between two halves of scratch
    const long long first = (n + kRedThreads - 1) / kRedThreads;
    if (first > 1 && (scratch == nullptr || 2 * first > scratch_floats))
        return hipErrorInvalidValue;
    const float *in = x;
    long long len = n;
    int side = 0;
    while (true) {
        const long long blocks = (len + kRedThreads - 1) / kRedThreads;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        float *dst = blocks == 1 ? out : scratch + side * first;
        reduce_tree_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kRedThreads), 0, stream>>>(
            in, len, dst);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || blocks == 1) return e;
        in = dst;
        len = blocks;
        side ^= 1;
    }
}

}  // namespace mgemm
