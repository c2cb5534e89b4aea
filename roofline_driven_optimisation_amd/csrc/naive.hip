// The unoptimised starting point: one thread per output element.
//
// Page "Naive GEMM and Roofline analysis", section 10.2: each thread walks k
// and accumulates A[row][k] * B[k][col]; threadIdx.x runs along columns so a
// wavefront's B reads are contiguous (section 10.3.2 explains why the other
// mapping is several times slower); blocks are 16 x 16 threads.  Unlike the
// page's listing this one applies the full alpha/beta update, accepts bf16
// inputs, flattens the grid to one dimension and can apply the fused
// bias / activation epilogue.  Its per-thread arithmetic
// intensity is 2K / (8K + 4), about 1/4 FLOP per byte, so it is left far
// below the roofline on purpose.
#include "common.h"
#include "kernels.h"

namespace mgemm {

namespace {

__device__ __forceinline__ float load_elem(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t *p, size_t i) {
    return bf16_bits_to_float(p[i]);
}

template <typename T, bool EPI>
__global__ __launch_bounds__(256) void naive_kernel(int M, int N, int K, float alpha, float beta,
                                                    const T *__restrict__ A,
                                                    const T *__restrict__ B, float *C,
                                                    int tiles_n, Epi epi) {
    const int tile = blockIdx.x;
    const int row = (tile / tiles_n) * 16 + threadIdx.y;
    const int col = (tile % tiles_n) * 16 + threadIdx.x;
    if (row >= M || col >= N) return;
    const T *a = A + static_cast<size_t>(row) * K;
    const T *b = B + col;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum = fmaf(load_elem(a, k), load_elem(b, static_cast<size_t>(k) * N), sum);
    const size_t idx = static_cast<size_t>(row) * N + col;
    float out = alpha * sum;
    if (beta != 0.0f) out = fmaf(beta, C[idx], out);
    C[idx] = epi_apply<EPI>(out, EPI && epi.bias ? epi.bias[col] : 0.0f, epi.act);
}

// An 8-bit float byte as fp32, from the format definitions: fmt 0 E4M3
// (bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, S.1111.111 NaN, no
// infinity), fmt 1 E5M2 (bias 15, 2 mantissa bits, subnormals m/4 * 2^-14,
// exponent 31 infinity or NaN).  Every value is exact in fp32.
__device__ __forceinline__ float fp8_to_float(uint8_t b, int fmt) {
    const bool neg = (b & 0x80u) != 0;
    float v;
    if (fmt == 0) {
        const uint32_t e = (b >> 3) & 15u, m = b & 7u;
        if (e == 15u && m == 7u) return __builtin_nanf("");
        v = e == 0u ? static_cast<float>(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    } else {
        const uint32_t e = (b >> 2) & 31u, m = b & 3u;
        if (e == 31u) return m == 0u ? (neg ? -__builtin_inff() : __builtin_inff()) : __builtin_nanf("");
        v = e == 0u ? static_cast<float>(m) * 0x1p-16f : __uint_as_float(((e + 112u) << 23) | (m << 21));
    }
    return neg ? -v : v;
}

// The 8-bit float fallback: one thread per output, B stored N x K.
__global__ __launch_bounds__(256) void naive_fp8_kernel(int M, int N, int K, float alpha,
                                                        float beta, const uint8_t *A,
                                                        const uint8_t *B, float *C, int tiles_n,
                                                        int fmt) {
    const int tile = blockIdx.x;
    const int row = (tile / tiles_n) * 16 + threadIdx.y;
    const int col = (tile % tiles_n) * 16 + threadIdx.x;
    if (row >= M || col >= N) return;
    const uint8_t *a = A + static_cast<size_t>(row) * K;
    const uint8_t *b = B + static_cast<size_t>(col) * K;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum = fmaf(fp8_to_float(a[k], fmt), fp8_to_float(b[k], fmt), sum);
    const size_t idx = static_cast<size_t>(row) * N + col;
    float out = alpha * sum;
    if (beta != 0.0f) out = fmaf(beta, C[idx], out);
    C[idx] = out;
}

// The batched fallback: item blockIdx.y, B stored K x N, or N x K with TRANSB.
template <bool TRANSB>
__global__ __launch_bounds__(256) void naive_batched_kernel(int M, int N, int K, float alpha,
                                                            float beta, const uint16_t *A,
                                                            const uint16_t *B, float *C,
                                                            int tiles_n, Batch batch) {
    const long long item = blockIdx.y;
    A += item * batch.stride_a;
    B += item * batch.stride_b;
    C += item * batch.stride_c;
    const int tile = blockIdx.x;
    const int row = (tile / tiles_n) * 16 + threadIdx.y;
    const int col = (tile % tiles_n) * 16 + threadIdx.x;
    if (row >= M || col >= N) return;
    const uint16_t *a = A + static_cast<size_t>(row) * K;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) {
        const size_t bi = TRANSB ? static_cast<size_t>(col) * K + k : static_cast<size_t>(k) * N + col;
        sum = fmaf(bf16_bits_to_float(a[k]), bf16_bits_to_float(B[bi]), sum);
    }
    const size_t idx = static_cast<size_t>(row) * N + col;
    float out = alpha * sum;
    if (beta != 0.0f) out = fmaf(beta, C[idx], out);
    C[idx] = out;
}

template <bool EPI>
__global__ __launch_bounds__(256) void scale_kernel(size_t count, int N, float beta, float *C,
                                                    Epi epi) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float v = (beta != 0.0f) ? beta * C[i] : 0.0f;
        C[i] = epi_apply<EPI>(v, EPI && epi.bias ? epi.bias[i % N] : 0.0f, epi.act);
    }
}

__global__ __launch_bounds__(256) void zero_ints_kernel(int *p, int count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

template <typename T>
hipError_t launch_naive(int M, int N, int K, float alpha, float beta, const T *A, const T *B,
                        float *C, const Epi &epi, hipStream_t stream) {
    const long long tiles_m = (M + 15) / 16, tiles_n = (N + 15) / 16;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tiles)), block(16, 16);
    if (epi_on(epi))
        naive_kernel<T, true><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                          static_cast<int>(tiles_n), epi);
    else
        naive_kernel<T, false><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                           static_cast<int>(tiles_n), epi);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_naive_f32(int M, int N, int K, float alpha, float beta, const float *A,
                            const float *B, float *C, const Epi &epi, hipStream_t stream) {
    return launch_naive<float>(M, N, K, alpha, beta, A, B, C, epi, stream);
}

hipError_t launch_naive_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                             const uint16_t *B, float *C, const Epi &epi, hipStream_t stream) {
    return launch_naive<uint16_t>(M, N, K, alpha, beta, A, B, C, epi, stream);
}

hipError_t launch_naive_bf16_batched(int M, int N, int K, float alpha, float beta,
                                     const uint16_t *A, const uint16_t *B, float *C,
                                     const Batch &batch, bool trans_b, hipStream_t stream) {
    const long long tiles_m = (M + 15) / 16, tiles_n = (N + 15) / 16;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL || batch.items < 1 || batch.items > 65535)
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(batch.items)),
        block(16, 16);
    if (trans_b)
        naive_batched_kernel<true><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                               static_cast<int>(tiles_n), batch);
    else
        naive_batched_kernel<false><<<grid, block, 0, stream>>>(M, N, K, alpha, beta, A, B, C,
                                                                static_cast<int>(tiles_n), batch);
    return hipGetLastError();
}

hipError_t launch_naive_fp8(int M, int N, int K, float alpha, float beta, const uint8_t *A,
                            const uint8_t *B, float *C, int fmt, hipStream_t stream) {
    const long long tiles_m = (M + 15) / 16, tiles_n = (N + 15) / 16;
    const long long tiles = tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL || (fmt != 0 && fmt != 1)) return hipErrorInvalidValue;
    naive_fp8_kernel<<<dim3(static_cast<unsigned>(tiles)), dim3(16, 16), 0, stream>>>(
        M, N, K, alpha, beta, A, B, C, static_cast<int>(tiles_n), fmt);
    return hipGetLastError();
}

hipError_t launch_scale_c(int M, int N, float beta, float *C, const Epi &epi,
                          hipStream_t stream) {
    const size_t count = static_cast<size_t>(M) * N;
    size_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (epi_on(epi))
        scale_kernel<true><<<grid, block, 0, stream>>>(count, N, beta, C, epi);
    else
        scale_kernel<false><<<grid, block, 0, stream>>>(count, N, beta, C, epi);
    return hipGetLastError();
}

hipError_t launch_zero_ints(int *p, int count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    zero_ints_kernel<<<dim3((count + 255) / 256), dim3(256), 0, stream>>>(p, count);
    return hipGetLastError();
}

}  // namespace mgemm
