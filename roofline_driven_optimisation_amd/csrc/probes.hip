// Measurement probes: the two hands-on exercises at the end of page "Memory
// hierarchy and cost table" (section 4.8), rebuilt for gfx950.
//
//   * Device-memory bandwidth test (the device-to-device leg of the
//     exercise): every 16-byte chunk of a buffer is read once, or read and
//     written to a second buffer.  Thread t of workgroup b reads chunks
//     t + 256 b + s u (s = 256 x grid, u = 0, 1, ...), eight loads in
//     flight per lane, so at every step the whole grid streams one
//     contiguous region: the flattest access pattern there is (the
//     coalescing rule of section 4.5.1 at grid scale).  The read form XORs
//     the words it reads, so the loads cannot be dropped, and each
//     workgroup writes its XOR to its own output word (no atomics, nothing
//     to wait on); the XOR of all output words is the XOR of every 32-bit
//     word of the buffer, which a test can check exactly.  Its time is the
//     practical ceiling of any kernel that reads the same bytes once, such
//     as a decode GEMM's weights.
//   * LDS bank conflicts (section 4.3.2): every lane reads one 4-byte LDS
//     word per step at word lane * stride + step + 17 wave (all inside the
//     64 KB table).  gfx950's LDS
//     has 64 banks of 4 bytes; stride 1 touches 64 different banks per
//     wave, stride 2 puts two lanes on each bank, stride 64 all 64 lanes on
//     one bank (different words), so the time per step grows with the
//     number of lanes that share a bank.  Each workgroup writes the XOR of
//     the words its lanes read.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

__device__ __forceinline__ uint32_t fold_block(uint32_t x) {
    // XOR over the workgroup: within each wave, then the four waves via LDS
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t s_wave[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = x;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= s_wave[w];
    return r;
}

template <bool COPY>
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(
    const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, long long chunks,
    uint32_t *__restrict__ out) {
    const long long stride = static_cast<long long>(gridDim.x) * kProbeThreads;
    long long i = static_cast<long long>(blockIdx.x) * kProbeThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kProbeUnroll - 1) * stride < chunks; i += kProbeUnroll * stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            if constexpr (COPY)
                __builtin_nontemporal_store(v[u], dst + i + u * stride);
            else
                x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
    }
    for (; i < chunks; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        if constexpr (COPY)
            __builtin_nontemporal_store(v, dst + i);
        else
            x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if constexpr (!COPY) {
        const uint32_t r = fold_block(x);
        if (threadIdx.x == 0) out[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(kProbeThreads) void lds_probe_kernel(int stride, int steps,
                                                                  uint32_t *__restrict__ out) {
    __shared__ uint32_t lds[kLdsProbeWords];
    for (int i = threadIdx.x; i < kLdsProbeWords; i += kProbeThreads)
        lds[i] = static_cast<uint32_t>(i) * 2654435761u;
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // words base .. base + steps - 1 of this lane; the launcher has checked
    // that 63 stride + 51 + steps <= kLdsProbeWords
    const uint32_t base = lane * static_cast<uint32_t>(stride) + 17u * wave;
    // volatile LDS reads: one 4-byte read per lane and step, never merged
    // into wider reads (which would change the bank pattern measured)
    typedef const volatile __attribute__((address_space(3))) uint32_t lds_word;
    lds_word *v = (lds_word *)(lds) + base;  // a C cast is the address-space cast
    uint32_t x = 0;
    int s = 0;
    for (; s + 8 <= steps; s += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[s + u];
    }
    for (; s < steps; ++s) x ^= v[s];
    const uint32_t r = fold_block(x);
    if (threadIdx.x == 0) out[blockIdx.x] = r;
}

}  // namespace

hipError_t launch_stream_probe(const void *src, void *dst, long long bytes, uint32_t *out,
                               int blocks, hipStream_t stream) {
    if (blocks < 1 || bytes < 0 || (bytes & 15) != 0) return hipErrorInvalidValue;
    const long long chunks = bytes / 16;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    if (dst != nullptr)
        stream_probe_kernel<true><<<dim3(blocks), dim3(kProbeThreads), 0, stream>>>(
            s, static_cast<u32x4 *>(dst), chunks, out);
    else
        stream_probe_kernel<false><<<dim3(blocks), dim3(kProbeThreads), 0, stream>>>(
            s, nullptr, chunks, out);
    return hipGetLastError();
}

hipError_t launch_lds_probe(int stride, int steps, uint32_t *out, int blocks,
                            hipStream_t stream) {
    if (blocks < 1 || stride < 0 || steps < 0 ||
        63LL * stride + 51 + steps > kLdsProbeWords)
        return hipErrorInvalidValue;
    lds_probe_kernel<<<dim3(blocks), dim3(kProbeThreads), 0, stream>>>(stride, steps, out);
    return hipGetLastError();
}

}  // namespace mgemm
