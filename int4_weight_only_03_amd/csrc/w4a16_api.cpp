// C-ABI layer: argument validation, path dispatch, host quantizer, status text.
//
// The quantizer follows the pages' quantize_w4a16 ("The Quiet Commit: How a
// Single Documentation Edit Marks the Completion of a Major Engineering
// Milestone", section "The INT4 Milestone": symmetric, group 32, 8 nibbles
// per int32 along K, value = nibble - 8).  The pages do not print the scale or
// rounding rule; this file uses scale = max|w|/7 and q = clamp(rint(w/scale),
// -8, 7), each division an IEEE fp32 true division rounded to nearest even.
// It is compiled without FMA contraction or fast-math so that it is bit-exact
// with any IEEE implementation of the same steps.

#include "../../include/w4a16.h"
#include "w4a16_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// N: rows of W; NY: columns of Y (N, or N / 2 for the fused SwiGLU)
int validate_gemm(const float *X, const int32_t *qweight, const float *scales, float *Y,
                  int64_t M, int64_t N, int64_t K, int32_t group, int64_t NY = -1) {
  if (NY < 0) NY = N;
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (M > W4A16_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!X || !qweight || !scales || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(qweight, 16) || !aligned(scales, 4) || !aligned(Y, 4))
    return W4A16_ERR_ALIGN;
  const size_t bx = size_t(M) * size_t(K) * 4, bq = size_t(N) * size_t(K) / 2,
               bs = size_t(N) * size_t(K / W4A16_GROUP) * 4, by = size_t(M) * size_t(NY) * 4;
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, qweight, bq) || overlaps(Y, by, scales, bs))
    return W4A16_ERR_ARG;
  return W4A16_OK;
}

// Every launch helper reports hipGetLastError() after its launches.  That
// per-thread slot also holds the status of the caller's own earlier HIP calls
// (a non-sticky error left there by someone else's call would otherwise be
// reported as this call's failure), so it is cleared right before a launch.
// Sticky errors (a fault of earlier work) cannot be cleared and still surface.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int select_path(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 0 || N <= 0) return W4A16_PATH_GEMV;  // no-op shapes: nothing runs
  if (M > W4A16_MAX_M || N > W4A16_MAX_N) return W4A16_PATH_TILE_MX;  // refused by the GEMM
  return w4a16::skinny_preferred(int(M), int(N)) ? W4A16_PATH_GEMV : W4A16_PATH_TILE_MX;
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char *w4a16_status_str(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_ARG: return "invalid argument";
    case W4A16_ERR_SHAPE: return "unsupported shape (K must be a multiple of 32; extents within limits)";
    case W4A16_ERR_ALIGN: return "misaligned pointer (X, qweight: 16 bytes; scales, Y: 4 bytes)";
    case W4A16_ERR_NONFINITE: return "non-finite weight";
    case W4A16_ERR_HIP: return "HIP runtime error";
    case W4A16_ERR_IO: return "weight file cannot be read or written, or has the wrong size";
    case W4A16_ERR_SCRATCH: return "the call needs more than the library's fixed scratch";
    default: return "unknown status";
  }
}

int w4a16_select_path(int64_t M, int64_t N, int64_t K) { return select_path(M, N, K); }

int w4a16_gemm_path(const float *X, const int32_t *qweight, const float *scales, float *Y,
                    int64_t M, int64_t N, int64_t K, int32_t group, int32_t path, void *stream) {
  if (path != W4A16_PATH_AUTO && path != W4A16_PATH_GEMV && path != W4A16_PATH_TILE &&
      path != W4A16_PATH_GEMV_FMA && path != W4A16_PATH_TILE_MX)
    return W4A16_ERR_ARG;
  int st = validate_gemm(X, qweight, scales, Y, M, N, K, group);
  if (st != W4A16_OK || M == 0 || N == 0) return st;
  if (path == W4A16_PATH_AUTO) path = select_path(M, N, K);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_stale_hip_error();

  hipError_t e;
  switch (path) {
    case W4A16_PATH_GEMV:
      e = w4a16::launch_gemv(X, qweight, scales, Y, int(M), int(N), int(K), s);
      break;
    case W4A16_PATH_GEMV_FMA:
      e = w4a16::launch_gemv_fma(X, qweight, scales, Y, int(M), int(N), int(K), s);
      break;
    case W4A16_PATH_TILE_MX:
      e = w4a16::launch_tile_mx(X, qweight, scales, Y, int(M), int(N), int(K), s);
      break;
    default:
      e = w4a16::launch_tile(X, qweight, scales, Y, int(M), int(N), int(K), s);
  }
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_read_floor(const void *const *ptrs, const int64_t *bytes, int32_t n, int32_t threads,
                     int32_t loads, void *sink, void *stream) {
  if (!ptrs || !bytes || !sink || n < 1 || n > 4) return W4A16_ERR_ARG;
  if (threads < 64 || threads > 1024 || threads % 64 != 0) return W4A16_ERR_ARG;
  if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return W4A16_ERR_ARG;
  if (!aligned(sink, 4)) return W4A16_ERR_ALIGN;
  long b[4];
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i] || bytes[i] < 0) return W4A16_ERR_ARG;
    if (!aligned(ptrs[i], 16) || bytes[i] % 16 != 0) return W4A16_ERR_ALIGN;
    b[i] = long(bytes[i]);
  }
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_read_floor(ptrs, b, n, threads, loads,
                                          static_cast<unsigned *>(sink),
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm(const float *X, const int32_t *qweight, const float *scales, float *Y, int64_t M,
               int64_t N, int64_t K, int32_t group, void *stream) {
  return w4a16_gemm_path(X, qweight, scales, Y, M, N, K, group, W4A16_PATH_AUTO, stream);
}

int w4a16_gemm_swiglu(const float *X, const int32_t *qweight, const float *scales, float *Y,
                      int64_t M, int64_t F, int64_t K, int32_t group, void *stream) {
  if (F < 0 || F > W4A16_MAX_N / 2) return F < 0 ? W4A16_ERR_ARG : W4A16_ERR_SHAPE;
  int st = validate_gemm(X, qweight, scales, Y, M, 2 * F, K, group, F);
  if (st != W4A16_OK || M == 0 || F == 0) return st;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_gemv_swiglu(X, qweight, scales, Y, int(M), int(F), int(K),
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_grouped(const float *X, const int32_t *token_index, const int32_t *expert_offsets,
                       const int32_t *qweight, const float *scales, float *Y, int64_t T,
                       int64_t R, int64_t E, int64_t N, int64_t K, int32_t group, void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (T < 0 || R < 0 || E <= 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (T > W4A16_MAX_M || R > W4A16_MAX_M || E > 65535 || N > W4A16_MAX_N || K > W4A16_MAX_K)
    return W4A16_ERR_SHAPE;
  if (R == 0 || N == 0) return W4A16_OK;
  if (T == 0) return W4A16_ERR_ARG;  // slots but no tokens to read
  if (!X || !token_index || !expert_offsets || !qweight || !scales || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(qweight, 16) || !aligned(scales, 4) || !aligned(Y, 4) ||
      !aligned(token_index, 4) || !aligned(expert_offsets, 4))
    return W4A16_ERR_ALIGN;
  const size_t bx = size_t(T) * size_t(K) * 4, by = size_t(R) * size_t(N) * 4;
  const size_t bq = size_t(E) * size_t(N) * size_t(K) / 2;
  const size_t bs = size_t(E) * size_t(N) * size_t(K / W4A16_GROUP) * 4;
  const size_t bi = size_t(R) * 4, bo = size_t(E + 1) * 4;
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, qweight, bq) || overlaps(Y, by, scales, bs) ||
      overlaps(Y, by, token_index, bi) || overlaps(Y, by, expert_offsets, bo))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_grouped(X, token_index, expert_offsets, qweight, scales, Y,
                                       int(T), int(R), int(E), int(N), int(K),
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

size_t w4a16_grouped_pack_bytes(int64_t E, int64_t N, int64_t K) {
  if (E <= 0 || N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (E > 65535 || N > W4A16_MAX_N || K > W4A16_MAX_K) return 0;
  return w4a16::grouped_pack_bytes(int(E), int(N), int(K));
}

int w4a16_grouped_pack(const int32_t *qweight, const float *scales, int64_t E, int64_t N,
                       int64_t K, int32_t group, void *packed, size_t packed_bytes,
                       void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (E <= 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (E > 65535 || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (N == 0) return W4A16_OK;
  if (!qweight || !scales || !packed) return W4A16_ERR_ARG;
  if (!aligned(qweight, 16) || !aligned(scales, 4)) return W4A16_ERR_ALIGN;
  const size_t need = w4a16::grouped_pack_bytes(int(E), int(N), int(K));
  if (!aligned(packed, 16) || packed_bytes < need) return W4A16_ERR_ARG;
  const size_t bq = size_t(E) * size_t(N) * size_t(K) / 2;
  const size_t bs = size_t(E) * size_t(N) * size_t(K / W4A16_GROUP) * 4;
  if (overlaps(packed, need, qweight, bq) || overlaps(packed, need, scales, bs))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_grouped_pack(qweight, scales, packed, int(E), int(N), int(K),
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_grouped_packed(const float *X, const int32_t *token_index,
                              const int32_t *expert_offsets, const void *packed, float *Y,
                              int64_t T, int64_t R, int64_t E, int64_t N, int64_t K,
                              int32_t group, void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (T < 0 || R < 0 || E <= 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (T > W4A16_MAX_M || R > W4A16_MAX_M || E > 65535 || N > W4A16_MAX_N || K > W4A16_MAX_K)
    return W4A16_ERR_SHAPE;
  if (R == 0 || N == 0) return W4A16_OK;
  if (T == 0) return W4A16_ERR_ARG;
  if (!X || !token_index || !expert_offsets || !packed || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(Y, 4) || !aligned(token_index, 4) ||
      !aligned(expert_offsets, 4))
    return W4A16_ERR_ALIGN;
  if (!w4a16::grouped_packed_supported(int(T), int(R), int(E), int(N), int(K)))
    return W4A16_ERR_SHAPE;
  const size_t bx = size_t(T) * size_t(K) * 4, by = size_t(R) * size_t(N) * 4;
  const size_t bp = w4a16::grouped_pack_bytes(int(E), int(N), int(K));
  const size_t bi = size_t(R) * 4, bo = size_t(E + 1) * 4;
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, packed, bp) || overlaps(Y, by, token_index, bi) ||
      overlaps(Y, by, expert_offsets, bo))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_grouped_packed(X, token_index, expert_offsets, packed, Y, int(T),
                                              int(R), int(E), int(N), int(K),
                                              reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

size_t w4a16_repacked_bytes(int64_t N, int64_t K, int32_t group) {
  if (group != W4A16_GROUP) return 0;
  return w4a16_grouped_pack_bytes(1, N, K);
}

int w4a16_repack(const int32_t *qweight, const float *scales, void *packed, int64_t N, int64_t K,
                 int32_t group, void *stream) {
  // the grouped layout with a single expert; the caller provides at least
  // w4a16_repacked_bytes(N, K, group) bytes
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (N == 0) return W4A16_OK;
  if (!qweight || !scales || !packed) return W4A16_ERR_ARG;
  if (!aligned(qweight, 16) || !aligned(scales, 4) || !aligned(packed, 16)) return W4A16_ERR_ALIGN;
  const size_t need = w4a16::grouped_pack_bytes(1, int(N), int(K));
  const size_t bq = size_t(N) * size_t(K) / 2, bs = size_t(N) * size_t(K / W4A16_GROUP) * 4;
  if (overlaps(packed, need, qweight, bq) || overlaps(packed, need, scales, bs))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_grouped_pack(qweight, scales, packed, 1, int(N), int(K),
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_repacked(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                        int64_t K, int32_t group, void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (M > W4A16_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!X || !packed || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(Y, 4)) return W4A16_ERR_ALIGN;
  const size_t bx = size_t(M) * size_t(K) * 4, by = size_t(M) * size_t(N) * 4;
  const size_t bp = w4a16::grouped_pack_bytes(1, int(N), int(K));
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, packed, bp)) return W4A16_ERR_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_stale_hip_error();

  hipError_t e;
  if (w4a16::gemv_kernel(int(M), int(N), int(K)) == W4A16_GEMV_MFMA)
    e = w4a16::launch_gemv_mfma_packed(X, packed, Y, int(M), int(N), int(K), s);
  else if (w4a16::skinny_preferred(int(M), int(N)))
    e = w4a16::launch_skinny_repacked(X, packed, Y, int(M), int(N), int(K), s);
  else
    e = w4a16::launch_tile_mx_packed(X, packed, Y, int(M), int(N), int(K), s);
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

size_t w4a16_small_packed_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > W4A16_SMALL_MAX_M || N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (N > W4A16_MAX_N || K > W4A16_MAX_K) return 0;
  return w4a16::small_packed_workspace_bytes(int(M), int(N), int(K));
}

int w4a16_gemm_small_packed(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                            int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (M > W4A16_SMALL_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!X || !packed || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(Y, 4)) return W4A16_ERR_ALIGN;
  const size_t bx = size_t(M) * size_t(K) * 4, by = size_t(M) * size_t(N) * 4;
  const size_t bp = w4a16::grouped_pack_bytes(1, int(N), int(K));
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, packed, bp)) return W4A16_ERR_ARG;
  const size_t need = w4a16::small_packed_workspace_bytes(int(M), int(N), int(K));
  if (need > 0) {
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W4A16_ERR_ARG;
    if (overlaps(workspace, need, X, bx) || overlaps(workspace, need, packed, bp) ||
        overlaps(workspace, need, Y, by))
      return W4A16_ERR_ARG;
  }
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_small_packed(X, packed, Y, int(M), int(N), int(K), workspace,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_small_packed_noalloc(const float *X, const void *packed, float *Y, int64_t M,
                                    int64_t N, int64_t K, int32_t group, void *stream) {
  static_assert(W4A16_NOALLOC_SCRATCH_BYTES == w4a16::kNoAllocScratchBytes, "scratch size");
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (M > W4A16_SMALL_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!X || !packed || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(Y, 4)) return W4A16_ERR_ALIGN;
  const size_t bx = size_t(M) * size_t(K) * 4, by = size_t(M) * size_t(N) * 4;
  const size_t bp = w4a16::grouped_pack_bytes(1, int(N), int(K));
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, packed, bp)) return W4A16_ERR_ARG;
  const size_t need = w4a16::small_packed_workspace_bytes(int(M), int(N), int(K));
  if (need > W4A16_NOALLOC_SCRATCH_BYTES) return W4A16_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0 && w4a16::noalloc_scratch(&ws) != hipSuccess) return W4A16_ERR_HIP;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_small_packed(X, packed, Y, int(M), int(N), int(K), ws,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemv_kernel(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (M > W4A16_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return 0;
  return w4a16::gemv_kernel(int(M), int(N), int(K));
}

int w4a16_grouped_kernel(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K) {
  if (T <= 0 || R <= 0 || E <= 0 || N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (T > W4A16_MAX_M || R > W4A16_MAX_M || E > 65535 || N > W4A16_MAX_N || K > W4A16_MAX_K)
    return 0;
  return w4a16::grouped_kernel(int(T), int(R), int(E), int(N), int(K));
}

size_t w4a16_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (M > W4A16_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return 0;
  return w4a16::split_workspace_bytes(int(M), int(N), int(K));
}

int w4a16_gemm_split(const float *X, const int32_t *qweight, const float *scales, float *Y,
                     int64_t M, int64_t N, int64_t K, int32_t group, void *workspace,
                     size_t workspace_bytes, void *stream) {
  int st = validate_gemm(X, qweight, scales, Y, M, N, K, group);
  if (st != W4A16_OK || M == 0 || N == 0) return st;
  const size_t need = w4a16::split_workspace_bytes(int(M), int(N), int(K));
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W4A16_ERR_ARG;
  const size_t bx = size_t(M) * size_t(K) * 4, bq = size_t(N) * size_t(K) / 2,
               bs = size_t(N) * size_t(K / W4A16_GROUP) * 4, by = size_t(M) * size_t(N) * 4;
  if (overlaps(workspace, need, X, bx) || overlaps(workspace, need, qweight, bq) ||
      overlaps(workspace, need, scales, bs) || overlaps(workspace, need, Y, by))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_split(X, qweight, scales, Y, int(M), int(N), int(K), workspace,
                                     reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

size_t w4a16_split_pack_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % W4A16_GROUP != 0) return 0;
  if (N > W4A16_MAX_N || K > W4A16_MAX_K) return 0;
  return w4a16::split_pack_bytes(int(N), int(K));
}

int w4a16_split_pack(const int32_t *qweight, const float *scales, int64_t N, int64_t K,
                     int32_t group, void *packed, size_t packed_bytes, void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (N == 0) return W4A16_OK;
  if (!qweight || !scales || !packed) return W4A16_ERR_ARG;
  if (!aligned(qweight, 16) || !aligned(scales, 4)) return W4A16_ERR_ALIGN;
  const size_t need = w4a16::split_pack_bytes(int(N), int(K));
  if (!aligned(packed, 16) || packed_bytes < need) return W4A16_ERR_ARG;
  const size_t bq = size_t(N) * size_t(K) / 2, bs = size_t(N) * size_t(K / W4A16_GROUP) * 4;
  if (overlaps(packed, need, qweight, bq) || overlaps(packed, need, scales, bs))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_split_pack(qweight, scales, packed, int(N), int(K),
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_gemm_split_packed(const float *X, const void *packed, float *Y, int64_t M, int64_t N,
                            int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (M < 0 || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (M > W4A16_MAX_M || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (!X || !packed || !Y) return W4A16_ERR_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(Y, 4)) return W4A16_ERR_ALIGN;
  const size_t bx = size_t(M) * size_t(K) * 4, by = size_t(M) * size_t(N) * 4;
  const size_t bp = w4a16::split_pack_bytes(int(N), int(K));
  if (overlaps(Y, by, X, bx) || overlaps(Y, by, packed, bp)) return W4A16_ERR_ARG;
  const size_t need = w4a16::split_workspace_bytes(int(M), int(N), int(K));
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W4A16_ERR_ARG;
  if (overlaps(workspace, need, X, bx) || overlaps(workspace, need, packed, bp) ||
      overlaps(workspace, need, Y, by))
    return W4A16_ERR_ARG;
  clear_stale_hip_error();

  hipError_t e = w4a16::launch_split_packed(X, packed, Y, int(M), int(N), int(K), workspace,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_quantize(const float *W, int32_t *qweight, float *scales, int64_t N, int64_t K,
                   int32_t group) {
  if (group != W4A16_GROUP) return W4A16_ERR_ARG;
  if (N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
  if (N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (N == 0) return W4A16_OK;
  if (!W || !qweight || !scales) return W4A16_ERR_ARG;
  const size_t total = size_t(N) * size_t(K);
  for (size_t i = 0; i < total; ++i)
    if (!std::isfinite(W[i])) return W4A16_ERR_NONFINITE;

  const int64_t G = K / W4A16_GROUP;
  for (int64_t n = 0; n < N; ++n) {
    const float *wrow = W + size_t(n) * size_t(K);
    uint32_t *qrow = reinterpret_cast<uint32_t *>(qweight) + size_t(n) * size_t(K / 8);
    for (int64_t g = 0; g < G; ++g) {
      const float *w = wrow + g * W4A16_GROUP;
      float amax = 0.0f;
      for (int i = 0; i < W4A16_GROUP; ++i) amax = std::fmax(amax, std::fabs(w[i]));
      volatile float seven = 7.0f;  // keep a true division, never a reciprocal multiply
      const float scale = amax / seven;
      scales[size_t(n) * size_t(G) + size_t(g)] = scale;
      uint32_t words[W4A16_GROUP / 8] = {0, 0, 0, 0};
      for (int i = 0; i < W4A16_GROUP; ++i) {
        float q = 0.0f;
        if (scale != 0.0f) {
          const float ratio = w[i] / scale;   // fp32 true division
          q = std::nearbyint(ratio);          // default mode: nearest, ties to even
          if (q < -8.0f) q = -8.0f;
          if (q > 7.0f) q = 7.0f;
        }
        const uint32_t nib = uint32_t(int(q) + 8);
        words[i / 8] |= nib << (4 * (i % 8));
      }
      std::memcpy(qrow + g * (W4A16_GROUP / 8), words, sizeof(words));
    }
  }
  return W4A16_OK;
}

}  // extern "C"
