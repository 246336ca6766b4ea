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
 * allocates nothing and keeps no state between calls, apart from the fixed
 * device scratch array of w4a16_gemm_small_packed_noalloc; every other entry
 * point is safe to call from several host threads at once.  Results of calls
 * that write the same Y buffer concurrently are undefined.
 *
 * Errors: argument problems are detected on the host, synchronously, before
 * anything is launched, and reported as a status code (Y untouched).  Work is
 * enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 * A launch that the HIP runtime refuses returns W4A16_ERR_HIP; faults that
 * happen later surface at the caller's next synchronisation.  Before it
 * launches, an entry point clears HIP's per-thread error slot, so that an
 * error left there by the caller's own earlier HIP calls is not reported as
 * this call's (sticky errors of earlier faults cannot be cleared and do).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 2
#define W4A16_GROUP 32

/* Largest supported extents.  M and N are limited so that grid indices fit in
 * 32 bits.  K is limited by accuracy: every kernel accumulates in fp32 (the
 * pages' choice for fidelity, "The Silence of Success: A Single Line That
 * Speaks Volumes", section "Assumptions Embedded in the Code"), and the
 * rounding error of its longest summation chain grows with K.  With
 * sign-coherent products (every x*w >= 0, the case where errors do not
 * cancel) the longest chain of any kernel stays within the tolerance
 * |dY| <= 1e-5 * sum|x*w| + 1e-6 up to K = 2^17 with a wide margin (the worst
 * is the per-group chain of the matrix-core kernels, about 0.3 of the
 * tolerance at K = 2^17); the tiled kernel adds its products in blocks of
 * 8 groups for that reason.  Larger K is refused with W4A16_ERR_SHAPE. */
#define W4A16_MAX_M ((int64_t)0x7fffffff)
#define W4A16_MAX_N ((int64_t)0x7fffffff)
#define W4A16_MAX_K ((int64_t)1 << 17)

/* Status codes (the int every entry point returns). */
#define W4A16_OK 0
#define W4A16_ERR_ARG 1       /* NULL pointer, negative extent, K == 0, group != 32,
                                 Y overlapping an input, unknown path */
#define W4A16_ERR_SHAPE 2     /* K % 32 != 0, or an extent above its W4A16_MAX_* */
#define W4A16_ERR_ALIGN 3     /* X or qweight not 16-byte aligned, scales or Y not
                                 4-byte aligned */
#define W4A16_ERR_NONFINITE 4 /* w4a16_quantize: a weight is NaN or infinite */
#define W4A16_ERR_HIP 5       /* the HIP runtime refused a launch */
#define W4A16_ERR_IO 6        /* w4a16_load_quantized / w4a16_save_quantized: a file cannot be
                                 opened, read or written, or its size is not the expected one */
#define W4A16_ERR_SCRATCH 7   /* w4a16_gemm_small_packed_noalloc: the call needs more scratch
                                 than the library's fixed W4A16_NOALLOC_SCRATCH_BYTES */

/* Kernel paths behind w4a16_gemm. */
#define W4A16_PATH_AUTO 0     /* what w4a16_gemm uses: w4a16_select_path() */
#define W4A16_PATH_GEMV 1     /* decode/verify path: dequant-on-the-fly kernels (the decode
                                 GEMVs, the skinny kernel at any M); which one:
                                 w4a16_gemv_kernel */
#define W4A16_PATH_TILE 2     /* tiled path: fp32 MFMA 32x32x2 on dequantized tiles */
#define W4A16_PATH_SPLIT 3    /* split-precision path (w4a16_gemm_split only): fp16 MFMA on
                                 exact (q - 8) codes and two fp16 limbs of each activation */
#define W4A16_PATH_GEMV_FMA 4 /* the fp32 FMA GEMV kernels for any M and K: one fp32 FMA per
                                 weight with the activations in VGPRs; for measurement beside
                                 the matrix-core GEMV (never the automatic choice) */
#define W4A16_PATH_TILE_MX 5  /* large-M matrix-core tile: fp16 MFMA 16x16x32 on exact (q - 8)
                                 codes and two fp16 limbs of each activation, prescaled by a
                                 power of two per row and pair of groups inside the kernel
                                 (the skinny kernel's arithmetic); 128 x 128 tiles, no
                                 workspace */

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
 * As w4a16_gemm, but with the kernel path forced (W4A16_PATH_AUTO, _GEMV,
 * _TILE, _GEMV_FMA or _TILE_MX; W4A16_PATH_SPLIT needs a workspace and is refused here
 * with W4A16_ERR_ARG).  Every path accepts every valid shape.  For tests and
 * measurement.
 */
int w4a16_gemm_path(const float *X, const int32_t *qweight, const float *scales, float *Y,
                    int64_t M, int64_t N, int64_t K, int32_t group, int32_t path,
                    void *stream);

/*
 * One-time repack of one weight matrix into a layout private to this
 * library's kernels, and the GEMM on it (the pages describe no repack; the
 * production kernel they plan to swap in brings layout and alignment
 * constraints of its own, "The Quiet Commit: How a Single Documentation Edit
 * Marks the Completion of a Major Engineering Milestone", section
 * "Assumptions and Potential Mistakes").  The repack moves bits only and is
 * meant to run once per weight, outside any timed or latency-critical path.
 *
 * The layout is that of w4a16_grouped_pack with one expert (E = 1): for
 * 16-row tile t and 4-group step s (S4 = ceil(K/128) steps), block
 * b = t*S4 + s holds 64 chunks of 16 bytes, chunk c + 16 R = word R of groups
 * 4s..4s+3 of row 16t + c, and then, after all T16*S4 kilobytes of weights,
 * the block's 16 x 4 scales (float (b*16 + c)*4 + q = scale of group 4s + q
 * of row 16t + c).  Rows past N and groups past K/32 hold 0x88888888 (weight
 * 0) and scale 0.  Every weight load of the kernels on it reads whole
 * kilobytes already in matrix-instruction operand order.
 */

/* Bytes of the repacked weights of an N x K matrix: ceil(N/16) * ceil(K/128)
 * * 1280 (qweight plus scales up to the padding of N to 16 rows and of the
 * group count to a multiple of 4).  0 if the shape or group is invalid.
 * Host only. */
size_t w4a16_repacked_bytes(int64_t N, int64_t K, int32_t group);

/* Repack qweight[N][K/8] and scales[N][K/32] (DEVICE memory) into `packed`
 * (DEVICE memory owned by the caller, 16-byte aligned, at least
 * w4a16_repacked_bytes(N, K, group) bytes, overlapping neither input).
 * Enqueued on `stream`.  N == 0 is a no-op; W4A16_ERR_ARG for a NULL or
 * overlapping pointer, negative extents, K == 0 or group != 32;
 * W4A16_ERR_ALIGN for a misaligned qweight (16 bytes), scales (4) or packed
 * (16); W4A16_ERR_SHAPE if K % 32 != 0 or an extent exceeds its limit. */
int w4a16_repack(const int32_t *qweight, const float *scales, void *packed, int64_t N,
                 int64_t K, int32_t group, void *stream);

/* Y[M][N] = X[M][K] . dequant(W)^T with W repacked by w4a16_repack(..., N, K,
 * ...).  No workspace and no allocation: where w4a16_gemv_kernel picks
 * W4A16_GEMV_MFMA, that decode GEMV, each lane gathering its group's 16 bytes
 * from four repacked chunks (bit for bit the result of w4a16_gemm on the
 * public layout); otherwise,
 * where w4a16_select_path picks the GEMV path, the kernel of W4A16_GEMV_SKINNY
 * reading the repacked blocks whole (limbs prescaled per row and pair of
 * groups, low limb x2^11), and where it picks W4A16_PATH_TILE_MX that
 * matrix-core tile on the repacked chunks (bit for bit its result on the
 * public layout).  All on the fp16
 * matrix instructions with exact weight codes and fp32 accumulation (a row of
 * X holding Inf or NaN gives non-finite values in that row of Y), within the
 * tolerance of w4a16_gemm, and deterministic.  X (16-byte aligned), packed
 * (16-byte aligned) and Y (4-byte aligned) are DEVICE memory; Y must not
 * overlap X or packed.
 * M == 0 or N == 0 is a no-op; otherwise errors as w4a16_gemm. */
int w4a16_gemm_repacked(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                        int64_t K, int32_t group, void *stream);

/*
 * Fused gate/up projection with a SwiGLU epilogue, for the decode MLP whose
 * gate and up projections share one W4A16 matrix ("gate+up (2x2048)" in the
 * pages' decode configuration; SwiGLU is the engine's MLP activation):
 * qweight[2F][K/8] and scales[2F][K/32] hold the gate rows 0..F-1 followed by
 * the up rows F..2F-1, and
 *     Y[m][j] = silu(g) * u,  g = X[m] . gate_j,  u = X[m] . up_j,
 *     silu(g) = g / (1 + exp(-g)),
 * with g and u the same fp32 group-scaled sums as w4a16_gemm and the epilogue
 * in fp32.  Y is [M][F] (not 2F); the gate/up outputs never reach memory.
 * Runs on the kernel w4a16_gemv_kernel(M, 2F, K) names: the matrix-core
 * decode GEMV, or else the skinny kernel's fused form (any M accepted: each
 * workgroup computes the gate and the up tiles of the same 16 x 32 or 16 x 16
 * outputs and stores the product).
 * Errors as w4a16_gemm with N = 2F.
 */
int w4a16_gemm_swiglu(const float *X, const int32_t *qweight, const float *scales, float *Y,
                      int64_t M, int64_t F, int64_t K, int32_t group, void *stream);

/*
 * Grouped (mixture-of-experts) W4A16 GEMM in one launch: many experts, each
 * applied to its own, possibly empty, set of token rows -- the pages run the
 * MoE experts through the INT4 path and plan a MoE kernel for production.
 *   X              float [T][K]        tokens
 *   token_index    int32 [R]           routed slot r reads token token_index[r]
 *   expert_offsets int32 [E+1]         expert e owns slots [offsets[e], offsets[e+1]):
 *                                      non-decreasing, offsets[0] = 0, offsets[E] = R
 *   qweight        int32 [E][N][K/8]   expert e's weights, layout as w4a16_gemm
 *   scales         float [E][N][K/32]
 *   Y              float [R][N]        Y[r] = X[token_index[r]] . dequant(W_e)^T, e
 *                                      the expert owning slot r
 * All DEVICE memory.  The kernel depends on the shape
 * (w4a16_grouped_kernel): on the matrix cores the arithmetic is that of
 * w4a16_gemm_split (exact weight codes, two fp16 limbs of each prescaled
 * activation, fp32 accumulation; a token row holding Inf or NaN gives NaN in
 * its slots' outputs); otherwise fp32 FMA as w4a16_gemm.  Either way the
 * tolerance of w4a16_gemm holds.  The weights of an expert with no slot are
 * not read.  token_index and expert_offsets are read on the device and
 * clamped into range (malformed routing gives wrong values, never an
 * out-of-bounds access).  R == 0 or N == 0 is a no-op; T == 0 with R > 0,
 * E < 1 or E > 65535 is an error; otherwise errors as w4a16_gemm (Y
 * overlapping any input is W4A16_ERR_ARG; token_index and expert_offsets
 * 4-byte aligned).
 */
int w4a16_gemm_grouped(const float *X, const int32_t *token_index, const int32_t *expert_offsets,
                       const int32_t *qweight, const float *scales, float *Y, int64_t T,
                       int64_t R, int64_t E, int64_t N, int64_t K, int32_t group, void *stream);

/*
 * Bytes of the packed expert weights w4a16_grouped_pack writes for E experts
 * of N x K (0 if the shape is invalid): E * ceil(N/16) * ceil(K/128) * 1280,
 * the size of qweight plus scales up to the padding of N to 16 rows and of
 * the group count to a multiple of 4.
 */
size_t w4a16_grouped_pack_bytes(int64_t E, int64_t N, int64_t K);

/*
 * One-time repack of expert weights qweight[E][N][K/8] and scales[E][N][K/32]
 * (DEVICE memory, the layouts of w4a16_gemm_grouped) into the grouped matrix-
 * core kernel's private layout, `packed` (DEVICE memory owned by the caller,
 * 16-byte aligned, at least w4a16_grouped_pack_bytes(E, N, K) bytes,
 * overlapping no input): a one-time repack into a layout private to this
 * library's kernels (the pages describe no repack; the production kernel
 * they plan to swap in brings layout and alignment constraints of its own,
 * "The Quiet Commit: How a Single Documentation Edit Marks the Completion of
 * a Major Engineering Milestone", section "Assumptions and Potential
 * Mistakes"); bits are moved only.  Layout, for
 * expert e, 16-row tile t (T16 = ceil(N/16) tiles) and 4-group step s
 * (S4 = ceil(K/128) steps), block b = (e*T16 + t)*S4 + s:
 *   bytes [0, E*T16*S4*1024): at b*64 + l chunks of 16 bytes, l = c + 16 R:
 *     word R of groups 4s, 4s+1, 4s+2, 4s+3 of row 16t + c;
 *   then E*T16*S4*256 bytes: at float (b*16 + c)*4 + q, the scale of group
 *     4s + q of row 16t + c.
 * Rows past N and groups past K/32 hold the word 0x88888888 (every code 8,
 * weight 0) and scale 0.  Every weight load of the packed GEMM then reads
 * whole contiguous kilobytes.  Enqueued on `stream`.  N == 0 is a no-op;
 * errors as w4a16_gemm_grouped (W4A16_ERR_ARG for a NULL, misaligned, too
 * small or overlapping `packed`).
 */
int w4a16_grouped_pack(const int32_t *qweight, const float *scales, int64_t E, int64_t N,
                       int64_t K, int32_t group, void *packed, size_t packed_bytes, void *stream);

/*
 * w4a16_gemm_grouped on weights packed by w4a16_grouped_pack(..., E, N, K,
 * ...): the same result, bit for bit, as w4a16_gemm_grouped on the unpacked
 * weights when that runs the matrix-core kernel (W4A16_GROUPED_MFMA), which
 * is the only kernel with a packed form: shapes for which
 * w4a16_grouped_kernel is not W4A16_GROUPED_MFMA return W4A16_ERR_SHAPE.
 * Otherwise errors as w4a16_gemm_grouped (`packed` 16-byte aligned, Y
 * overlapping it is W4A16_ERR_ARG).
 */
int w4a16_gemm_grouped_packed(const float *X, const int32_t *token_index,
                              const int32_t *expert_offsets, const void *packed, float *Y,
                              int64_t T, int64_t R, int64_t E, int64_t N, int64_t K,
                              int32_t group, void *stream);

/*
 * Small-M GEMM on packed weights: Y[M][N] = X[M][K] . dequant(W)^T for
 * 1 <= M <= W4A16_SMALL_MAX_M, W packed once by w4a16_grouped_pack(qweight,
 * scales, 1, N, K, ...) (a single expert).  For the pages' tree-verification
 * batches (a few dozen draft tokens scored against each weight in one pass).
 * The arithmetic of w4a16_gemm_split (exact weight codes, two fp16 limbs of
 * each activation, fp32 accumulation; a row of X holding Inf or NaN gives NaN
 * in that row of Y), within the tolerance of w4a16_gemm; each row's power of
 * two is taken per K slice.  The K range may be split over workgroups; their
 * partial results go to `workspace` and are added in a fixed order
 * (deterministic).  workspace: DEVICE memory of at least
 * w4a16_small_packed_workspace_bytes(M, N, K) bytes, 256-byte aligned, not
 * overlapping X, packed or Y; it may be NULL when that size is 0.  Its contents
 * on entry do not matter and are clobbered.  X, packed (16-byte aligned) and Y
 * are DEVICE memory; Y must not overlap X or packed.  M == 0 or N == 0 is a
 * no-op; M > W4A16_SMALL_MAX_M is W4A16_ERR_SHAPE; a missing, misaligned, too
 * small or overlapping workspace is W4A16_ERR_ARG; otherwise errors as
 * w4a16_gemm.
 */
#define W4A16_SMALL_MAX_M 64
int w4a16_gemm_small_packed(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                            int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Workspace bytes w4a16_gemm_small_packed needs (0 when K is not split, or
 * when the shape is not accepted).  Host only. */
size_t w4a16_small_packed_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * w4a16_gemm_small_packed for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels, the same plan and the same result bit for
 * bit, with the split-K partials in a scratch array the library holds in
 * device memory instead of a caller workspace.  The array is
 * W4A16_NOALLOC_SCRATCH_BYTES per device, a file-scope device variable that
 * each GPU the library runs on keeps until the process ends (its address is
 * looked up once per device, on the first call there); no call allocates or
 * frees anything.  Every call on one GPU shares that GPU's array and leaves
 * its last partials there: calls that may overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  A shape
 * whose partials, w4a16_small_packed_workspace_bytes(M, N, K), exceed
 * W4A16_NOALLOC_SCRATCH_BYTES is refused with W4A16_ERR_SCRATCH before any GPU
 * work; otherwise arguments and errors as w4a16_gemm_small_packed (no
 * workspace arguments).
 */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w4a16_gemm_small_packed_noalloc(const float *X, const void *packed, float *Y, int64_t M,
                                    int64_t N, int64_t K, int32_t group, void *stream);

/* Kernels behind w4a16_gemm_grouped. */
#define W4A16_GROUPED_MFMA 1  /* matrix cores, split-path arithmetic; up to 4096 experts
                                 and the token rows of a slot chunk staged in LDS */
#define W4A16_GROUPED_ROWS 2  /* fp32 FMA, token rows staged in LDS */
#define W4A16_GROUPED_GEMV 3  /* fp32 FMA, activations read from memory */

/* The kernel w4a16_gemm_grouped runs for T tokens, R slots, E experts and an
 * N x K expert shape (one of W4A16_GROUPED_*), or 0 for a shape it refuses or
 * treats as a no-op.  Host only; no GPU use. */
int w4a16_grouped_kernel(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K);

/* Kernels behind W4A16_PATH_GEMV. */
#define W4A16_GEMV_MFMA 1     /* M <= 4, and 5 <= M <= 8 unless N >= 4096 and K >= 4096 (any
                                 K; beyond 8192, 8 waves take blocks of 16 groups in turn):
                                 v_mfma_f32_4x4x4_16b_f16 on exact weight
                                 codes (nibble - 8) and two fp16 limbs of each activation; every
                                 group of 32 activations is scaled by a power of two (max |x|
                                 into [2^14, 2^15)) before the split, so the limbs hold 22
                                 significant bits of every activation down to 2^-28 of its
                                 group's maximum (the low limb carried x2^11); products exact
                                 in fp32, fp32 accumulation, one fp32 multiply per (row,
                                 group) applies scale * 2^-e */
#define W4A16_GEMV_FMA 2      /* the fp32 FMA GEMV (one fp32 FMA per weight, activations in
                                 VGPRs): no longer returned for any shape; it runs under
                                 W4A16_PATH_GEMV_FMA */
#define W4A16_GEMV_SKINNY 3   /* M >= 9 (the tree-verification batches and beyond), and
                                 5 <= M <= 8 when N >= 4096 and K >= 4096:
                                 v_mfma_f32_16x16x32_f16 on exact weight codes and two fp16
                                 limbs of each activation, prescaled by a power of two per
                                 row and pair of groups, the low limb x2^11 and met by the
                                 codes x2^-11; fp32 accumulation; 16 rows of X by 16-64 rows
                                 of W per workgroup, whose 8 waves split K in steps of 4
                                 groups and add their partial tiles in order; no workspace */

/* The kernel W4A16_PATH_GEMV runs for an M x N x K shape (one of W4A16_GEMV_*), or 0
 * for a shape w4a16_gemm refuses.  Host only; no GPU use.  (Decode GEMV: the pages'
 * path for memory-bound MoE inference, "The Quiet Commit: How a Single Plan Update
 * Closed Phase 3 of a Native DDTree Inference Engine", section "Input and Output
 * Knowledge".) */
int w4a16_gemv_kernel(int64_t M, int64_t N, int64_t K);

/* The path W4A16_PATH_AUTO takes for this shape (W4A16_PATH_GEMV or _TILE_MX): the
 * GEMV path for M <= 64; above that the cheaper of the skinny kernel and the
 * 128 x 128 matrix-core tile by rounds over 256 compute units, each weighted by
 * its workgroup's measured cost: ceil(ceil(M/16) * ceil(N/(16 NT)) / 256) * NT
 * for the skinny kernel (NT = 4, 2 or 1 column tiles of 16, the widest that
 * leaves at least 256 workgroups) against ceil(ceil(M/128) * ceil(N/128) / 256)
 * * 33 for the tile, the skinny kernel on a tie.  The fp32 tiled path
 * (W4A16_PATH_TILE) is no longer chosen: the skinny kernel is about twice as
 * fast on every shape where the tile does not win.  For M or N <= 0 (no-ops)
 * the GEMV path, for M or N beyond W4A16_MAX_M / W4A16_MAX_N (refused by the
 * GEMM) the tile.  Host only; no GPU use. */
int w4a16_select_path(int64_t M, int64_t N, int64_t K);

/*
 * Workspace bytes w4a16_gemm_split needs for this shape (0 if the shape is
 * invalid).  It holds the activation limbs (4*M*K bytes), per-row exponents,
 * split-K partial tiles and counters.
 */
size_t w4a16_split_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Y = X . dequant(qweight, scales)^T on the fp16 matrix cores with fp32
 * accumulation: each weight code (nibble - 8) is exact in fp16; each row of X is
 * scaled by a power of two (max |x| into [2^14, 2^15)) and split into two fp16
 * limbs hi = f16(x'), lo = f16(x' - hi); the products are exact in fp32 and
 * accumulated in fp32, one fp32 FMA per group applies the group scale, and the
 * row's power of two is undone exactly at the store.  A second kernel-side
 * reading of the same operation the pages define (fp32 activations, int4
 * weights, fp32 accumulation), for compute-bound shapes.
 *
 * Range: the limbs hold 22 significant bits of every activation down to about
 * 2^-17 of its row's largest magnitude; smaller ones keep an absolute error
 * below 2^-39 of that maximum (the low limb reaches the fp16 subnormals).  The
 * tolerance of w4a16_gemm holds for rows whose magnitudes span up to about
 * 2^22; a row spanning 2^26 or more whose largest entries meet zero weights
 * can leave it.  The same holds for the other entry points on this arithmetic
 * (w4a16_gemm_split_packed, w4a16_gemm_grouped(_packed),
 * w4a16_gemm_small_packed(_noalloc), the last per row and K slice).
 * w4a16_gemm's own limb kernels (W4A16_GEMV_MFMA, W4A16_GEMV_SKINNY,
 * W4A16_PATH_TILE_MX), which w4a16_gemm_repacked runs as well, take a power
 * of two per row and one or two groups of 32 and carry the low limb x2^11,
 * which keeps the tolerance for rows spanning 2^30 and more.
 *
 * `workspace` is a DEVICE buffer owned by the caller, 256-byte aligned, of at
 * least w4a16_split_workspace_bytes(M, N, K) bytes, not overlapping any other
 * argument; its contents need no initialisation and are scratch on return.
 * Two calls that share a workspace must not run concurrently.  Enqueues two
 * kernels on `stream`.  Errors as w4a16_gemm, plus W4A16_ERR_ARG for a NULL,
 * misaligned, too small or overlapping workspace.
 */
int w4a16_gemm_split(const float *X, const int32_t *qweight, const float *scales, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t group, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Bytes of the packed weights w4a16_split_pack writes for an N x K matrix
 * (0 if the shape is invalid): ceil(N/64) * ceil(K/64) * 2560 bytes, the same
 * as qweight plus scales up to the padding of N to 64 rows and of the group
 * count to even.
 */
size_t w4a16_split_pack_bytes(int64_t N, int64_t K);

/*
 * One-time repack of qweight[N][K/8] and scales[N][K/32] (DEVICE memory, the
 * layouts above) into the split path's kernel-private layout, `packed` (DEVICE
 * memory owned by the caller, 16-byte aligned, at least
 * w4a16_split_pack_bytes(N, K) bytes, overlapping no input): a one-time
 * repack into a layout private to this library's kernels (as for
 * w4a16_grouped_pack); it moves bits only (the weights and scales are copied
 * unchanged).  Layout,
 * for slab s of 64 rows and stage t of 2 groups (S = ceil(N/64) slabs,
 * T = ceil(K/64) stages):
 *   bytes [0, S*T*2048): at ((s*T + t)*2 + g)*64 + r chunks of 16 bytes, the
 *     4 words of group 2t+g of row 64s+r;
 *   then S*T*512 bytes: at float index (s*T + t)*128 + 2r + g, its scale.
 * Rows past N and the group past K/32 (K/32 odd) hold words 0x88888888 (code
 * 0) and scale 0.  Enqueued on `stream`; errors as w4a16_gemm (W4A16_ERR_ARG
 * for a NULL, misaligned, too small or overlapping `packed`).
 */
int w4a16_split_pack(const int32_t *qweight, const float *scales, int64_t N, int64_t K,
                     int32_t group, void *packed, size_t packed_bytes, void *stream);

/*
 * w4a16_gemm_split on weights packed by w4a16_split_pack(..., N, K, ...):
 * the same result, bit for bit, as w4a16_gemm_split on the unpacked weights,
 * with every weight and scale copy reading whole cache lines.  Workspace as
 * for w4a16_gemm_split (w4a16_split_workspace_bytes(M, N, K)).  X must not
 * overlap Y; `packed` is 16-byte aligned.
 */
int w4a16_gemm_split_packed(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                            int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Raw weight files of one quantized weight W[N][K], as the pages' INT4 model
 * bundles store them: "<name>.qw" holds qweight[N][K/8] as little-endian int32
 * and "<name>.sc" holds scales[N][K/32] as little-endian fp32, both row-major
 * with no header; the group size (32) is metadata kept apart from the files,
 * and a weight with a .qw file runs through W4A16 while the others stay fp32
 * ("The Quiet Commit: How a Single Documentation Edit Marks the Completion of
 * a Major Engineering Milestone", section "The INT4 Milestone: From FP32 to
 * Production-Ready Quantization").  The files carry no shape, so the caller
 * passes N and K; each file must be exactly N*K/2 (.qw) and N*K/8 (.sc) bytes.
 *
 * w4a16_load_quantized reads both files into HOST buffers the caller owns
 * (qweight: N*K/8 int32, scales: N*K/32 float).  Synchronous; no GPU use.
 * Returns W4A16_ERR_IO if a file cannot be opened or read or has another size
 * (both sizes are checked before anything is read; on any error the buffers'
 * contents are unspecified), W4A16_ERR_NONFINITE if a scale is NaN or
 * infinite (the quantizer writes none), W4A16_ERR_ARG on NULL
 * paths or buffers, negative extents, K == 0 or group != 32, W4A16_ERR_SHAPE
 * if K % 32 != 0 or an extent exceeds its W4A16_MAX_*.  N == 0 reads two empty
 * files.
 */
int w4a16_load_quantized(const char *qw_path, const char *sc_path, int64_t N, int64_t K,
                         int32_t group, int32_t *qweight, float *scales);

/*
 * Write qweight[N][K/8] and scales[N][K/32] (HOST memory) to the two raw files
 * above, replacing any existing files.  Synchronous.  Errors as
 * w4a16_load_quantized (W4A16_ERR_IO when a file cannot be written).
 */
int w4a16_save_quantized(const char *qw_path, const char *sc_path, int64_t N, int64_t K,
                         int32_t group, const int32_t *qweight, const float *scales);

/*
 * Measurement helper, not part of the GEMM: one launch that streams n <= 4
 * DEVICE segments ptrs[i] (16-byte aligned) of bytes[i] bytes (multiples of
 * 16; host arrays of n entries) with `loads` nontemporal 16-byte loads per
 * thread (1, 2, 4, 8 or 16, all issued before any is used) and `threads`
 * threads per block (64..1024, a multiple of 64), and writes at most one
 * word to `sink` (DEVICE, 4 bytes).  A benchmark times it over the buffers a
 * GEMM call reads (X, qweight, scales) to measure the streaming-read ceiling
 * of one launch of that size.  Enqueued on `stream`; W4A16_ERR_ARG for bad
 * counts, shapes or NULL pointers, W4A16_ERR_ALIGN for misaligned segments or
 * sizes.
 */
int w4a16_read_floor(const void *const *ptrs, const int64_t *bytes, int32_t n, int32_t threads,
                     int32_t loads, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
