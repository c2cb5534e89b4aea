// Host-side launchers of the kernels, used by the C ABI in gemm_api.hip.
// Every launcher enqueues work on `stream` and returns the launch status;
// shapes and pointers have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgemm {

// Fused Linear-layer epilogue, applied after alpha and beta:
// C = act(alpha * A * B + beta * C + bias[n]).  Every launcher takes one;
// {nullptr, kActNone} is the plain GEMM, and kernels are instantiated without
// the epilogue code for it.
enum Activation { kActNone = 0, kActRelu = 1, kActGelu = 2, kActSilu = 3 };
struct Epi {
    const float *bias;  // N fp32 values in device memory, or nullptr
    int act;            // an Activation
};
inline bool epi_on(const Epi &e) { return e.bias != nullptr || e.act != kActNone; }
constexpr Epi kNoEpi = {nullptr, kActNone};

// Strided batch of independent GEMMs: item b uses A + b stride_a, B + b
// stride_b and C + b stride_c (elements).  {1, 0, 0, 0} is a single GEMM.
struct Batch {
    int items;
    long long stride_a, stride_b, stride_c;
};
constexpr Batch kOneItem = {1, 0, 0, 0};

// One thread per output element (the unoptimised starting point).
hipError_t launch_naive_f32(int M, int N, int K, float alpha, float beta, const float *A,
                            const float *B, float *C, const Epi &epi, hipStream_t stream);
hipError_t launch_naive_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                             const uint16_t *B, float *C, const Epi &epi, hipStream_t stream);

// C = act(beta * C + bias) (beta * C, or zeros when beta == 0, without an
// epilogue): the K == 0 case.
hipError_t launch_scale_c(int M, int N, float beta, float *C, const Epi &epi,
                          hipStream_t stream);

// Fill `count` ints with zero (workspace counters).
hipError_t launch_zero_ints(int *p, int count, hipStream_t stream);

// fp32 LDS-tiled fp32-MFMA kernel.  `vec` selects 16-byte accesses, which
// need K % 4 == 0, N % 4 == 0 and 16-byte aligned A, B and C.
hipError_t launch_f32_mfma(int M, int N, int K, float alpha, float beta, const float *A,
                           const float *B, float *C, bool vec, const Epi &epi,
                           hipStream_t stream);
const char *f32_mfma_name(bool vec);

// bf16 LDS-tiled MFMA kernel.  Needs K % 8 == 0, N % 8 == 0, 16-byte
// aligned A and B, K <= 2^21 and N <= 2^20.  `cfg` indexes the tile table.
struct Bf16TileConfig {
    int bm, bn;
    const char *name;
};
int bf16_num_tile_configs();
const Bf16TileConfig &bf16_tile_config(int cfg);
// `allow_split`: a 256 x 256 kernel may split its last round (see PPSplit).
int bf16_pick_tile_config(int M, int N, int K, int num_cus, bool allow_split);

// Split of a 256 x 256 kernel's trailing tiles over K (the four-wave, the
// ping-pong and the 8-bit float kernel share the scheme and the layout of
// the partials).  When the tile count leaves a last round at most half full,
// its r tiles are each computed by two workgroups, one per part of the K
// steps: the first posts its partial sums, the second adds them and writes
// C, so the last round takes about half as long on twice as many CUs.
//
// The pair's handshake.  When a workgroup of a pair starts, one thread swaps
// the epoch into the tile's claim word: the first to claim (old value !=
// epoch) becomes split 0, takes the first split_step K steps, posts its
// partial tile and then publishes the epoch in the tile's flag with a
// release store; the other becomes split 1, takes the remaining steps,
// waits for the flag with an acquire, adds the partial to its own sums and
// writes C.  The waiting workgroup thus only ever waits for one that is
// already running and never waits itself, whatever order the workgroups
// were dispatched in.  The wait is bounded by poll_limit flag reads; a wait
// that gives up writes NaN into its tile and adds one to *timeouts, which
// the host can read back.
constexpr int kPPTile = 256;  // the square tile of both 256 x 256 kernels
constexpr int kPollLimitDefault = 1 << 22;  // flag reads, about 0.5 s
struct PPSplit {
    int split_from;   // tiles at or past this position in the order are split
    int split_step;   // first K step (of 32) of the second half
    float *partials;  // one kPPTile^2 fp32 tile per split tile
    unsigned *flags;  // one word per split tile, never equal to epoch on entry
    unsigned *claims; // one word per split tile, never equal to epoch on entry
    unsigned epoch;   // a value flags and claims have not held before this launch
    // 0: workgroups 2i and 2i + 1 share a tile (different XCDs); partials,
    // flags and claims must be uncached memory and their accesses are
    // system-scope.  1: workgroups b and b + 8 share a tile, which puts both
    // on one XCD on a device that deals workgroups to its eight XCDs in
    // round-robin order (probe_xcd_mapping checks this); partials, flags and
    // claims are ordinary device memory that no other XCD uses during the
    // launch, their accesses are device-scope, and the number of split tiles
    // is a multiple of 8.
    int xcd_pairs;
    int grid_tiles;      // set by the launcher: the tile count
    int poll_limit;      // flag reads before a waiting workgroup gives up
    unsigned *timeouts;  // uncached word counting waits that gave up (may be null)
};
int bf16_pp_config();                                          // the ping-pong tile index
bool bf16_config_splits(int cfg);  // the 256 x 256 kernels, which can split a last round
const char *bf16_split_name(int cfg, bool xcd_pairs);  // kernel name of a split launch
int bf16_pp_split_tiles(int M, int N, int K, int num_cus);    // 0: no split
hipError_t launch_bf16_mfma(int cfg, int M, int N, int K, float alpha, float beta,
                            const uint16_t *A, const uint16_t *B, float *C, const PPSplit *split,
                            const Epi &epi, hipStream_t stream);
// Strided batched bf16 GEMM on the tiled kernels, no split and no fused
// epilogue: `cfg` 0 (the four-wave 256 x 256 kernel), 3 (128 x 128) or 5
// (the four-wave kernel on 16 x 16 MFMAs), each with B as K x N or stored
// transposed, N x K (trans_b); `staged` (cfg 3 only) stores C through LDS;
// `persist_grid` (cfg 0 only, a multiple of 8, 0 for none) runs that many
// workgroups, each over every grid-th tile, when there are more tiles;
// `stages` other than 2 (B as K x N only): 128 x 128 tiles (cfg 3) on 4 LDS
// stages or 256 x 128 tiles (cfg 1) on 3, copies that many K steps less one
// ahead.  The same shape requirements as launch_bf16_mfma, for every item
// (strides keep each item 16-byte aligned).
hipError_t launch_bf16_batched(int cfg, int M, int N, int K, float alpha, float beta,
                               const uint16_t *A, const uint16_t *B, float *C, const Batch &batch,
                               bool trans_b, hipStream_t stream, bool staged = false,
                               int persist_grid = 0, int stages = 2);
// 8-bit float GEMM, C = alpha A B^T + beta C with B stored N x K: fmt 0
// E4M3, 1 E5M2 (both operands).  Needs K % 16 == 0, 16-byte aligned A and
// B, K <= 2^21 and N <= 2^20.  `wide`: the 128-deep K step kernel, else the
// 64-deep one.  `split` (or null) splits tiles as for the bf16 256 x 256
// kernels, with split_step counted in the kernel's K steps.
constexpr int kFp8BK = 64;        // bytes (= elements) per K step
constexpr int kFp8WideBK = 128;   // the same for the 128-deep kernel
hipError_t launch_fp8_gemm(int M, int N, int K, float alpha, float beta, const uint8_t *A,
                           const uint8_t *B, float *C, int fmt, const PPSplit *split,
                           hipStream_t stream, bool wide);
// Tiles of an fp8 GEMM worth splitting over K (its last round when at most
// half full and K has at least 8 steps of `bk`), else 0.
int fp8_split_tiles(int M, int N, int K, int num_cus, int bk);
// One thread per output element for any 8-bit float shape or alignment.
hipError_t launch_naive_fp8(int M, int N, int K, float alpha, float beta, const uint8_t *A,
                            const uint8_t *B, float *C, int fmt, hipStream_t stream);

// One thread per output element, any layout: the batched fallback.
hipError_t launch_naive_bf16_batched(int M, int N, int K, float alpha, float beta,
                                     const uint16_t *A, const uint16_t *B, float *C,
                                     const Batch &batch, bool trans_b, hipStream_t stream);

// Skinny-M (M <= 16) bf16 kernel that streams B once from HBM.  Needs
// K % 8 == 0, N % 8 == 0 and 16-byte aligned A, B and C.  With splits > 1 the
// K range is divided over `splits` workgroups per column block, which reduce
// through `partials` (splits * M * N floats) and `counters` (`counter_ints`
// ints, at least one per column block, zero on entry and left zero on
// exit); both must live in uncached device memory (hipDeviceMallocUncached).
constexpr int kSkinnyMaxM = 16;
constexpr int kSkinnyCols = 128;  // output columns per workgroup
// Split count for the decode shapes; `xcd_local` picks the rule for the
// XCD-local reduction (launch_skinny_bf16_xcd), whose partials are cheaper.
int skinny_pick_splits(int M, int N, int K, int num_cus, bool xcd_local);
// Whether each K-slice of B (and all of A) stays below 2^31 bytes, the reach
// of the kernel's 32-bit buffer offsets, with `splits` slices.
bool skinny_slice_fits(int M, int N, int K, int splits);
hipError_t launch_skinny_bf16(int M, int N, int K, float alpha, float beta, const uint16_t *A,
                              const uint16_t *B, float *C, int splits, float *partials,
                              int *counters, int counter_ints, const Epi &epi,
                              hipStream_t stream);

// Split-K skinny kernel with most of its reduction kept inside XCDs.  On a
// device that deals workgroups to its eight XCDs in round-robin order, so
// that ids equal modulo 8 share an XCD (probe_xcd_mapping checks this),
// the first 8 * floor(col_blocks / 8) column blocks are placed so that all
// splits of a block share one XCD and reduce through its L2, in ordinary
// (cached) device memory: `xcd_base` is kXcdCount blocks of kSkinnyXcdBytes,
// block x touched only by the workgroups with blockIdx % 8 == x, each holding
// kSkinnyXcdCounterInts counters (zero on entry and left zero on exit) and
// then the partial sums (xcd_block_bytes per block in all).  The remaining
// col_blocks % 8 column blocks reduce through `partials` and `counters` as
// in launch_skinny_bf16, unless all_local: then those blocks are XCD-local
// too (some XCDs get one block more, the grid is padded with workgroups
// that exit at once) and `partials` and `counters` are not used.
// skinny_xcd_local_fits says whether a shape may use this form.
constexpr int kXcdCount = 8;
constexpr size_t kSkinnyXcdBytes = size_t(4) << 20;
constexpr int kSkinnyXcdCounterInts = 16384;
bool skinny_xcd_local_fits(int M, int N, int K, int splits, size_t block_bytes, bool all_local);
hipError_t launch_skinny_bf16_xcd(int M, int N, int K, float alpha, float beta,
                                  const uint16_t *A, const uint16_t *B, float *C, int splits,
                                  float *partials, int *counters, int counter_ints,
                                  char *xcd_base, size_t xcd_block_bytes, int xcd_group,
                                  bool all_local, const Epi &epi, hipStream_t stream);
// Sum of a float32 vector (4-byte aligned, any length) into *out, on the
// device.  blocks <= kReduceMaxBlocks workgroups each stream a contiguous
// chunk; with blocks > 1 they reduce through `partials` (blocks floats) and
// `counter` (one int, zero on entry and left zero), both uncached memory.
constexpr int kReduceMaxBlocks = 2048;
long long reduce_blocks(long long n, int num_cus);
hipError_t launch_reduce_sum(const float *x, long long n, float *out, float *partials,
                             int *counter, int blocks, hipStream_t stream);
// The ladder's first rung: one element per thread, an LDS tree per 256,
// relaunched on its partials (two halves of `scratch`, ping-pong) until one
// value is left.  Needs 2 * ceil(n / 256) scratch floats when n > 256.
hipError_t launch_reduce_sum_tree(const float *x, long long n, float *out, float *scratch,
                                  long long scratch_floats, hipStream_t stream);

// Measurement probes (probes.hip).  launch_stream_probe reads `bytes`
// (a multiple of 16; src 16-byte aligned) with `blocks` workgroups of 256
// threads: dst == nullptr XORs the words and writes workgroup b's XOR to
// out[b] (`blocks` words); otherwise it copies src to dst (out unused).
// launch_lds_probe runs `steps` 4-byte LDS reads per lane at word
// lane * stride + step + 17 wave (63 stride + 51 + steps must not exceed
// kLdsProbeWords, else hipErrorInvalidValue) of a table holding
// word i = i * 2654435761 (mod 2^32), and writes workgroup b's XOR of
// what its lanes read to out[b].
constexpr int kLdsProbeWords = 16384;  // 64 KB of LDS
hipError_t launch_stream_probe(const void *src, void *dst, long long bytes, uint32_t *out,
                               int blocks, hipStream_t stream);
hipError_t launch_lds_probe(int stride, int steps, uint32_t *out, int blocks,
                            hipStream_t stream);

// Runs a probe grid on `stream`, waits for it, and sets *ok when every
// workgroups whose ids are equal modulo kXcdCount ran on one XCD and the
// kXcdCount residues on different XCDs (which XCD takes workgroup 0 varies
// between launches and is not checked).  The grid writes kXcdProbeInts ints
// into `buffer` (device memory the caller owns), or into a block the
// function allocates and frees when `buffer` is null.
constexpr int kXcdProbeInts = 4096;
hipError_t probe_xcd_mapping(bool *ok, hipStream_t stream, int *buffer = nullptr);

}  // namespace mgemm
