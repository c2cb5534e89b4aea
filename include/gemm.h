/*
 * gemm.h -- C ABI of libgemm.so, a GEMM library for AMD MI355X (gfx950).
 *
 * Operation (page "Naive GEMM and Roofline analysis", section 10.1, the GEMM
 * definition):
 *
 *     C[m][n] = alpha * sum_k A[m][k] * B[k][n] + beta * C[m][n]
 *
 * Layout.  Every matrix is dense and row-major with no padding, as in the
 * naive kernel of section 10.2 of that page: A is M x K (A[m][k] at m*K+k),
 * B is K x N (B[k][n] at k*N+n), C is M x N (C[m][n] at m*N+n).  There are no
 * transpose flags and no leading-dimension arguments.
 *
 * Pointers.  A, B and C are DEVICE pointers on the current HIP device.
 * ``stream`` is a hipStream_t passed as void* (NULL = the null stream).  Work
 * is enqueued on that stream and the call returns without waiting for it;
 * a fault inside a kernel surfaces at the caller's next synchronisation.
 *
 * Ownership.  The caller owns A, B, C and the stream.  A and B are only read.
 * C is read (only when beta != 0) and written in place.  C must not overlap A
 * or B.  The library keeps no pointer after the call returns.
 *
 * Special cases.  M == 0 or N == 0: returns GEMM_OK and launches nothing.
 * K == 0: C = beta * C (zeros when beta == 0).  beta == 0: C is never read, so
 * it may hold NaN or garbage.  Any shape and any pointer alignment is
 * accepted; fast vectorised kernels run when rows are 16-byte aligned, other
 * inputs go to slower kernels that load element by element.
 *
 * Workspace.  Two bf16 paths split K across workgroups and exchange partial
 * sums through a scratch area: the decode-shaped (skinny-M) kernel, and the
 * large-M kernel when its last round of 256 x 256 tiles would be at most half
 * full (gemm_fp8 splits such a round too, and reduce_sum_f32 uses the area
 * for its partial sums).  The library allocates the area lazily on the first
 * such call for a given (device, stream) pair and reuses it afterwards; it is
 * never freed before process exit.  It is 64 MiB + 128 KiB of uncached
 * device memory (hipExtMallocWithFlags), plus 96 MiB + 64 KiB of ordinary
 * device memory (hipMalloc) through which workgroups that share an XCD
 * exchange partial sums.  Before its first use of the latter on a device,
 * the library runs a small probe grid on the caller's stream and waits for
 * it, to check that the device deals workgroups to its eight XCDs in
 * round-robin order (ids equal modulo 8 share an XCD); where it does not,
 * both paths exchange through the uncached area alone.  At most sixteen
 * streams per device get an area (2.5 GiB at most): calls on further streams run
 * the same kernels without splitting K (slower on the shapes above, same
 * results within the tolerances; the vector sums return GEMM_ERR_ALLOC for
 * vectors long enough to need the area).  Concurrent calls on
 * different streams get different workspaces; concurrent calls from several
 * host threads on one stream must be serialised by the caller, as the
 * stream would serialise them anyway.  The fp32 path never uses a
 * workspace.
 *
 * Split pairs.  When a last round of 256 x 256 tiles is split, the two
 * workgroups of a tile exchange one partial tile: the one that starts first
 * takes the first part of K, posts its partial and publishes it with a
 * release store; the other takes the rest and waits for it with an acquire
 * (a bounded wait on a workgroup that is already running and never waits
 * itself).  If the wait ever gave up, the tile's C values are NaN and the
 * call has already returned GEMM_OK; gemm_split_timeouts() reports how many
 * waits gave up on a stream.
 *
 * Graph capture.  A call on a stream that is being captured into a HIP graph
 * allocates nothing, runs no probe and launches only kernels whose replays
 * are independent: the decode-shaped kernel splits K only if the capturing
 * stream already owns a workspace (from an earlier, uncaptured call on it;
 * the kernel leaves its counters re-armed), and the large-M kernel never
 * splits its last round (that split's flags are tagged with a per-call
 * number that a replay would reuse).  Replays of such a graph use the
 * capturing stream's workspace and must not overlap other calls on it.
 *
 * Errors.  No call aborts or throws across the ABI.  Negative sizes, or a
 * NULL pointer for a matrix with a non-zero number of elements, return
 * GEMM_ERR_INVALID_ARG and launch nothing.  A failed
 * launch returns GEMM_ERR_LAUNCH, a failed workspace allocation (or, for
 * the vector sums, no workspace to be had) GEMM_ERR_ALLOC and a failed
 * device query GEMM_ERR_DEVICE.
 */
#ifndef MI355X_GEMM_H
#define MI355X_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_ABI_VERSION 8

#if defined(__GNUC__) || defined(__clang__)
#define GEMM_API __attribute__((visibility("default")))
#else
#define GEMM_API
#endif

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,
    GEMM_ERR_LAUNCH = 2,
    GEMM_ERR_ALLOC = 3,
    GEMM_ERR_DEVICE = 4,
    GEMM_ERR_SCRATCH = 5  /* gemm_bf16_noalloc: the call needs more than its fixed scratch */
};

/*
 * fp32 GEMM: A, B and C are float32.  Products and sums are fp32 (matrix-core
 * fp32 MFMA on the tiled path); alpha and beta are applied in fp32 in the
 * kernel's epilogue.
 */
GEMM_API int gemm_f32(int M, int N, int K, float alpha, float beta,
             const float *A, const float *B, float *C, void *stream);

/*
 * bf16-input GEMM: A and B hold bf16 bit patterns (the upper 16 bits of an
 * IEEE binary32); C is float32 in and out.  Products are exact in fp32 and
 * are accumulated in fp32.  M <= 16 runs the HBM-streaming decode kernel,
 * larger M the LDS-tiled MFMA kernel.
 */
GEMM_API int gemm_bf16(int M, int N, int K, float alpha, float beta,
              const uint16_t *A, const uint16_t *B, float *C, void *stream);

/*
 * gemm_bf16 for callers that cannot allocate device memory: code running
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layouts, semantics and error behaviour as
 * gemm_bf16; this entry point calls no hipMalloc, hipFree or allocating
 * library routine.  Its only scratch is a fixed 8 MiB array in the
 * library's device code (one per GPU, held until the process ends): the
 * decode-shaped kernel (M <= 16) splits K through it, with every column
 * block's partial sums kept inside one XCD; other shapes run the tiled
 * kernel on whole tiles (no split of a last round).  A decode-shaped call
 * whose split would need more than the array holds returns GEMM_ERR_SCRATCH
 * and launches nothing: each XCD's 1 MiB share keeps 64 KiB of counters and
 * the fp32 partial sums of its ceil(N / 1024) column blocks of 128, so it
 * takes ceil(N / 1024) * splits * M <= 1920 (the decode shapes split K
 * eight ways: N = 11008 at M = 16 uses 1408; N = 16384 at M = 16 is
 * refused).
 * The first call on a device that is not under graph capture clears the
 * array's counters and, if no gemm_bf16 call has done so yet, runs the XCD
 * dealing probe (both on the caller's stream, waiting for the probe);
 * before that, and on a device that does not deal workgroups round-robin,
 * decode-shaped calls run in one split.  Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, or
 * host threads) race and must be serialised by the caller.
 */
GEMM_API int gemm_bf16_noalloc(int M, int N, int K, float alpha, float beta,
                               const uint16_t *A, const uint16_t *B, float *C, void *stream);

/*
 * Fused Linear-layer epilogue.  A Linear layer computes Y = XW + b (page
 * "From model computation to GPU execution", section 1.1), and fusing the
 * elementwise work that follows a GEMM into its epilogue keeps the
 * intermediate out of HBM (page "Where kernel performance comes from",
 * section on optimising memory-bound kernels).  These entry points compute
 *
 *     C = act(alpha * A * B + beta * C + bias[n])
 *
 * in the same kernels and with the same arguments, layouts, dispatch and
 * error behaviour as gemm_f32 / gemm_bf16, plus:
 *   bias        device pointer to N float32 values, one per column of C
 *               (read-only, caller-owned), or NULL for no bias;
 *   activation  one of enum gemm_activation, applied in fp32 after the bias:
 *               GEMM_ACT_NONE  x;
 *               GEMM_ACT_RELU  0 for x < 0, else x (NaN stays NaN);
 *               GEMM_ACT_GELU  x * Phi(x), Phi the standard normal CDF
 *                              (the erf form; Phi from the erf
 *                              approximation 7.1.26 of Abramowitz and
 *                              Stegun, absolute error <= 1.5e-7);
 *               GEMM_ACT_SILU  x / (1 + exp(-x)) (hardware exponential and
 *                              reciprocal).
 *               Any other value returns GEMM_ERR_INVALID_ARG and launches
 *               nothing.
 * With K == 0 the result is act(beta * C + bias) (zeros plus bias when beta
 * is 0).  bias == NULL with GEMM_ACT_NONE is exactly gemm_f32 / gemm_bf16.
 */
enum gemm_activation {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,
    GEMM_ACT_GELU = 2,
    GEMM_ACT_SILU = 3
};
GEMM_API int gemm_f32_bias_act(int M, int N, int K, float alpha, float beta,
                               const float *A, const float *B, float *C,
                               const float *bias, int activation, void *stream);
GEMM_API int gemm_bf16_bias_act(int M, int N, int K, float alpha, float beta,
                                const uint16_t *A, const uint16_t *B, float *C,
                                const float *bias, int activation, void *stream);

/*
 * The unoptimised starting point of section 10.2 of page "Naive GEMM and
 * Roofline analysis": one thread per output element, a plain loop over k,
 * 16 x 16 thread blocks, with the full alpha/beta update.  Same arguments and
 * semantics as gemm_f32 / gemm_bf16; kept as the first rung of the
 * optimisation ladder and as a correctness cross-check.
 */
GEMM_API int gemm_naive_f32(int M, int N, int K, float alpha, float beta,
                   const float *A, const float *B, float *C, void *stream);
GEMM_API int gemm_naive_bf16(int M, int N, int K, float alpha, float beta,
                    const uint16_t *A, const uint16_t *B, float *C, void *stream);

/*
 * 8-bit float GEMM: the smaller input type that raises the arithmetic
 * intensity (page "Where kernel performance comes from", section on GEMM:
 * one-byte operands move half the bytes of bf16 per multiply-add).
 *
 *     C = alpha * scale_a * scale_b * A * B^T + beta * C
 *
 * A is M x K and B is stored N x K (row n of B holds the K weights of
 * output column n), both row-major bytes in `format`: GEMM_FP8_E4M3 (bias 7,
 * 3 mantissa bits, largest 448, no infinity) or GEMM_FP8_E5M2 (bias 15, 2
 * mantissa bits, largest 57344); scale_a and scale_b are per-tensor scales.
 * Products are exact in fp32 and accumulate in fp32; C is float32 in and
 * out.  K % 16 == 0 with 16-byte aligned A and B runs the matrix-core
 * kernel (256 x 256 tiles, v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
 * scales), anything else a one-thread-per-output kernel.  As in gemm_bf16, a
 * last round of tiles that is at most half full is split over K through the
 * library's per-device workspace (allocated on first use: GEMM_ERR_ALLOC if
 * that fails; not split while the stream is being captured).  An unknown
 * format and the gemm_bf16 argument errors return GEMM_ERR_INVALID_ARG.
 */
enum gemm_fp8_format { GEMM_FP8_E4M3 = 0, GEMM_FP8_E5M2 = 1 };
GEMM_API int gemm_fp8(int M, int N, int K, float alpha, float beta, const uint8_t *A,
                      const uint8_t *B, float *C, float scale_a, float scale_b, int format,
                      void *stream);

/*
 * Strided batched bf16 GEMM, the shape attention gives the GEMM: S = Q K^T
 * and O = P V (page "From model computation to GPU execution", section
 * 1.2), one product per head (page "Naive GEMM and Roofline analysis",
 * section 10.1).  For b = 0 .. batch-1:
 *
 *     C_b = alpha * A_b * op(B_b) + beta * C_b
 *
 * A_b = A + b * stride_a is M x K row-major; B_b = B + b * stride_b is
 * K x N row-major (trans_b == 0, op = identity) or N x K row-major
 * (trans_b == 1, op = transpose: a key matrix stored token by token);
 * C_b = C + b * stride_c is M x N float32.  Strides count elements; A and B
 * strides may be 0 (one operand shared by every item), stride_c must be at
 * least M * N when batch > 1.  Device pointers, caller-owned, asynchronous.
 * Items run in one launch of the four-wave 256 x 256 kernel (or the
 * 128 x 128 one when N <= 128 and B is not transposed) when K % 8 == 0,
 * N % 8 == 0 (B not transposed), A and B are 16-byte aligned with strides
 * that are multiples of 8; otherwise a one-thread-per-output kernel.  No
 * split-K and no fused epilogue here.  batch < 0, batch > 65535, trans_b
 * not 0 or 1, negative strides, overlapping C items and the gemm_bf16
 * argument errors return GEMM_ERR_INVALID_ARG.
 */
GEMM_API int gemm_bf16_strided_batched(int batch, int M, int N, int K, float alpha, float beta,
                                       const uint16_t *A, int64_t stride_a,
                                       const uint16_t *B, int64_t stride_b, int trans_b,
                                       float *C, int64_t stride_c, void *stream);

/*
 * Sum of a float32 vector, the memory-bound case study of page "Memory
 * hierarchy and cost table", section 4.7 (summing 100 million floats):
 *
 *     *out = x[0] + x[1] + ... + x[n-1]
 *
 * x and out are device pointers (x: n floats, 4-byte aligned, read-only;
 * out: one float, written), owned by the caller.  Sums are fp32 in a fixed
 * order, so repeated calls give identical bits; no element passes through
 * more than n / 2^21 + 32 fp32 additions (reduce_sum_f32; ceil(log2 n) for
 * the naive form), which bounds the rounding error by that many units of
 * 2^-24 times sum |x|.  n == 0 writes 0.  Asynchronous like the GEMMs; negative n, a NULL out, a NULL x
 * with n > 0 or a misaligned x return GEMM_ERR_INVALID_ARG and launch
 * nothing.  Vectors longer than a few thousand floats are summed by
 * several workgroups through the stream's workspace (as the GEMMs' split-K
 * is); GEMM_ERR_ALLOC when no workspace can be had (graph capture on a
 * stream that has none, or more streams than the library keeps areas for).
 * reduce_sum_f32 is the optimised form (16-byte loads, one workgroup per
 * contiguous chunk); reduce_sum_f32_naive is the page's first version (one
 * element per thread, a shared-memory tree per 256 elements) with the
 * global atomic replaced by further tree passes; it can sum up to 2^31
 * elements.
 */
GEMM_API int reduce_sum_f32(const float *x, int64_t n, float *out, void *stream);
GEMM_API int reduce_sum_f32_naive(const float *x, int64_t n, float *out, void *stream);

/*
 * Measurement probes: the hands-on exercises that close page "Memory
 * hierarchy and cost table" (section 4.8), a device-to-device bandwidth test
 * and a shared-memory bank-conflict demonstration (section 4.3.2).  They
 * compute nothing of the GEMM; bench.py times them beside it.  Asynchronous
 * on `stream` like the GEMMs; every pointer is a device pointer owned by
 * the caller; `blocks` (1 .. 2^20) is the number of 256-thread workgroups.
 *
 * gemm_probe_stream reads the `bytes` bytes at src (a multiple of 16,
 * src 16-byte aligned) once, every 16-byte chunk with one load, the whole
 * grid streaming one contiguous region at a time.  dst == NULL: out (blocks
 * words) receives one XOR per workgroup, and the XOR of all of them is the
 * XOR of every 32-bit word of src.  dst != NULL (16-byte aligned, not
 * overlapping src): src is copied to dst and out is not used (may be NULL).
 * Its time is the practical floor of any kernel that reads (or copies) as
 * many bytes.
 *
 * gemm_probe_lds has every lane of each workgroup read `steps` 4-byte words
 * of a 64 KB shared-memory table whose word i holds i * 2654435761 (mod
 * 2^32): lane l of wave w reads words l * stride + 17 w + j, j = 0 .. steps
 * - 1, so `stride` sets how many lanes of a wave share one of the 64 banks
 * (1: none; 2: pairs; 64: all).  out (blocks words) receives, per
 * workgroup, the XOR of every word its lanes read.  63 stride + 51 + steps
 * must not exceed 16384.
 *
 * Argument errors (sizes, alignment, NULL where a pointer is needed) return
 * GEMM_ERR_INVALID_ARG and launch nothing.
 */
GEMM_API int gemm_probe_stream(const void *src, void *dst, int64_t bytes, uint32_t *out,
                               int blocks, void *stream);
GEMM_API int gemm_probe_lds(int stride, int steps, uint32_t *out, int blocks, void *stream);

/* Static English text for a gemm_status value (never NULL). */
GEMM_API const char *gemm_status_string(int status);

/*
 * Name of the kernel the most recent gemm_* call made on the calling host
 * thread launched ("none" if it launched nothing).  Static storage; valid
 * until the next call on the same thread.  For tests and benchmarks.
 */
GEMM_API const char *gemm_last_kernel(void);

/*
 * Name of the kernel that gemm_bf16 (is_bf16 != 0) or gemm_f32 (is_bf16 ==
 * 0) would launch for an M x N x K call on the current device, without
 * launching anything: the dispatch rule applied to the kernel signature and
 * launch configuration of page "Naive GEMM and Roofline analysis", section
 * 10.2 (which kernel, which grid, for a given M, N, K).  It assumes 16-byte
 * aligned A, B and C and a call on the null stream that is not being
 * captured, and reads the same MGEMM_* environment overrides as the calls.
 * Before the first call that needed the XCD probe on this device, it
 * assumes the probe passes.  Returns "none" for M == 0 or N == 0,
 * "scale_c" for K == 0, "invalid" for negative sizes or a failed device
 * query.  Static storage, never NULL.
 */
GEMM_API const char *gemm_kernel_name(int is_bf16, int M, int N, int K);

/*
 * Diagnostic: how many split-pair waits gave up (and wrote NaN into their
 * tile) on `stream` (current device) since the previous call; *count is set
 * to that number and the count is cleared.  Waits on `stream` first (it
 * copies the count back), so it must not be called while the stream is
 * being captured (GEMM_ERR_INVALID_ARG).  A stream without a workspace
 * reports 0.  NULL count: GEMM_ERR_INVALID_ARG.
 */
GEMM_API int gemm_split_timeouts(void *stream, long long *count);

/*
 * Test hooks.  They change how later calls behave, so that tests can reach
 * paths that normal inputs never take; every kernel still runs to its end.
 *   GEMM_TEST_POLL_LIMIT  the number of flag reads a split pair's second
 *                         workgroup makes before it gives up (value < 0
 *                         restores the default, about half a second's
 *                         worth; 0 makes every such wait give up at once);
 *                         process-wide; `stream` is ignored.
 *   GEMM_TEST_EPOCH       sets the last split epoch used on `stream`'s
 *                         workspace (current device) to (uint32_t)value, so
 *                         that a test can run calls across the point where
 *                         the 32-bit epoch wraps to zero (the library then
 *                         clears the flags on the stream and restarts at 1);
 *                         GEMM_ERR_INVALID_ARG if the stream has no
 *                         workspace yet.
 * An unknown hook returns GEMM_ERR_INVALID_ARG.
 */
enum gemm_test_hook_id { GEMM_TEST_POLL_LIMIT = 1, GEMM_TEST_EPOCH = 2 };
GEMM_API int gemm_test_hook(int hook, long long value, void *stream);

/* GEMM_ABI_VERSION of the built library. */
GEMM_API int gemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355X_GEMM_H */
