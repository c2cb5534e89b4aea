// Host-side launchers of the kernels, used by the C ABI in gemm_api.hip.
// Every launcher enqueues work on `stream` and returns the launch status;
// shapes and pointers have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgemm {

// One thread per output element (the unoptimised starting point).
hipError_t launch_naive_f32(int M, int N, int K, float alpha, float beta, const float *A,
                            const float *B, float *C, hipStream_t stream);
hipError_t launch_naive_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                             const uint16_t *B, float *C, hipStream_t stream);

// C = beta * C (zeros when beta == 0): the K == 0 case.
hipError_t launch_scale_c(int M, int N, float beta, float *C, hipStream_t stream);

// Fill `count` ints with zero (workspace counters).
hipError_t launch_zero_ints(int *p, int count, hipStream_t stream);

// fp32 LDS-tiled fp32-MFMA kernel.  `vec` selects 16-byte accesses, which
// need K % 4 == 0, N % 4 == 0 and 16-byte aligned A, B and C.
hipError_t launch_f32_mfma(int M, int N, int K, float alpha, float beta, const float *A,
                           const float *B, float *C, bool vec, hipStream_t stream);
const char *f32_mfma_name(bool vec);

// bf16 LDS-tiled MFMA kernel.  Needs K % 8 == 0, N % 8 == 0, 16-byte
// aligned A and B, K <= 2^21 and N <= 2^20.  `cfg` indexes the tile table.
struct Bf16TileConfig {
    int bm, bn;
    const char *name;
};
int bf16_num_tile_configs();
const Bf16TileConfig &bf16_tile_config(int cfg);
int bf16_pick_tile_config(int M, int N, int K, int num_cus);
hipError_t launch_bf16_mfma(int cfg, int M, int N, int K, float alpha, float beta,
                            const uint16_t *A, const uint16_t *B, float *C, hipStream_t stream);

// Skinny-M (M <= 16) bf16 kernel that streams B once from HBM.  Needs
// K % 8 == 0, N % 8 == 0 and 16-byte aligned A, B and C.  With splits > 1 the
// K range is divided over `splits` workgroups per column block, which reduce
// through `partials` (splits * M * N floats) and `counters` (`counter_ints`
// ints, at least one per column block, zero on entry and left zero on
// exit); both must live in uncached device memory (hipDeviceMallocUncached).
constexpr int kSkinnyMaxM = 16;
constexpr int kSkinnyCols = 128;  // output columns per workgroup
int skinny_pick_splits(int M, int N, int K, int num_cus);
hipError_t launch_skinny_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                              const uint16_t *B, float *C, int splits, float *partials,
                              int *counters, int counter_ints, hipStream_t stream);

}  // namespace mgemm
