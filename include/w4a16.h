/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 group-quantized GEMM library.
 *
 *     Y[M][N] = X[M][K] . dequant(qweight, scales)^T
 *
 * The operation is the one the pages name w4a16_gemm: fp32 activations times
 * int4 weights stored 8 nibbles per int32 along the input dimension, value =
 * nibble - 8, times one fp32 scale per group of 32 input columns, accumulated
 * in fp32 ("The Quiet Commit: How a Single Documentation Edit Marks the
 * Completion of a Major Engineering Milestone", section "The INT4 Milestone";
 * "The Silence of Success: A Single Line That Speaks Volumes", section "What
 * the Edit Actually Built").  The quantizer is the pages' quantize_w4a16
 * (same page and section): symmetric, one scale per group of 32.
 *
 * Layouts (all row-major, contiguous, no strides):
 *   X        float   [M][K]      row stride 4*K bytes
 *   qweight  int32   [N][K/8]    word j of row n holds k = 8j+i in bits 4i..4i+3,
 *                                i = 0..7, low nibble first; w = (nibble - 8) * scale
 *   scales   float   [N][K/32]   scale of group g = k/32 of row n
 *   Y        float   [M][N]
 *
 * Memory and ownership: every pointer argument of w4a16_gemm* is a DEVICE
 * pointer owned by the caller; w4a16_quantize takes HOST pointers.  The library
 * allocates nothing, keeps no state between calls and is safe to call from
 * several host threads at once.  Results of calls that write the same Y
 * buffer concurrently are undefined.
 *
 * Errors: argument problems are detected on the host, synchronously, before
 * anything is launched, and reported as a status code (Y untouched).  Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 * A launch that the HIP runtime refuses returns W4A16_ERR_HIP; faults that
 * happen later surface at the caller's next synchronisation.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1
#define W4A16_GROUP 32

/* Largest supported extents.  K is limited so that one row of X stays below
 * 2 GiB; M and N so that grid indices fit in 32 bits. */
#define W4A16_MAX_M ((int64_t)0x7fffffff)
#define W4A16_MAX_N ((int64_t)0x7fffffff)
#define W4A16_MAX_K ((int64_t)1 << 28)

/* Status codes (the int every entry point returns). */
#define W4A16_OK 0
#define W4A16_ERR_ARG 1       /* NULL pointer, negative extent, K == 0, group != 32,
                                 Y overlapping an input, unknown path */
#define W4A16_ERR_SHAPE 2     /* K % 32 != 0, or an extent above its W4A16_MAX_* */
#define W4A16_ERR_ALIGN 3     /* X or qweight not 16-byte aligned, scales or Y not
                                 4-byte aligned */
#define W4A16_ERR_NONFINITE 4 /* w4a16_quantize: a weight is NaN or infinite */
#define W4A16_ERR_HIP 5       /* the HIP runtime refused a launch */

/* Kernel paths behind w4a16_gemm. */
#define W4A16_PATH_AUTO 0     /* what w4a16_gemm uses: w4a16_select_path() */
#define W4A16_PATH_GEMV 1     /* decode/verify path: dequant-on-the-fly GEMV, x in VGPRs */
#define W4A16_PATH_TILE 2     /* tiled path: fp32 MFMA 32x32x2 on dequantized tiles */

/* Version of this ABI (W4A16_ABI_VERSION of the library that was built). */
int w4a16_abi_version(void);

/* Static text for a status code ("ok", "invalid argument", ...). Never NULL. */
const char *w4a16_status_str(int status);

/*
 * Quantize fp32 weights W[N][K] (HOST memory) into qweight[N][K/8] and
 * scales[N][K/32] (HOST memory, caller-allocated).  Per group of 32 along K:
 * scale = max|w| / 7 (fp32 division, round to nearest even); q = rint(w/scale)
 * with an fp32 division and ties to even, clamped to [-8, 7]; nibble = q + 8.
 * A group whose scale is 0 gets nibble 8 everywhere.  Synchronous, no GPU use.
 * Returns W4A16_ERR_NONFINITE (outputs untouched) if any weight is NaN or
 * infinite, W4A16_ERR_SHAPE if K % 32 != 0, W4A16_ERR_ARG on NULL pointers,
 * negative extents or group != 32.  N == 0 is a no-op.
 */
int w4a16_quantize(const float *W, int32_t *qweight, float *scales,
                   int64_t N, int64_t K, int32_t group);

/*
 * Y = X . dequant(qweight, scales)^T, fp32 accumulation; Y is overwritten (not
 * accumulated into).  group must be 32 and K a multiple of 32.  M == 0 or
 * N == 0 is a no-op that returns W4A16_OK without touching the GPU.  Y must not
 * overlap X, qweight or scales.  The kernel path is w4a16_select_path(M, N, K).
 */
int w4a16_gemm(const float *X, const int32_t *qweight, const float *scales, float *Y,
               int64_t M, int64_t N, int64_t K, int32_t group, void *stream);

/*
 * As w4a16_gemm, but with the kernel path forced (one of W4A16_PATH_*); every
 * path accepts every valid shape.  For tests and measurement.
 */
int w4a16_gemm_path(const float *X, const int32_t *qweight, const float *scales, float *Y,
                    int64_t M, int64_t N, int64_t K, int32_t group, int32_t path,
                    void *stream);

/* The path W4A16_PATH_AUTO takes for this shape (W4A16_PATH_GEMV or _TILE). */
int w4a16_select_path(int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
