// Internal interface between the C-ABI layer (w4a16_api.cpp) and the kernel
// translation units.  Arguments reaching these launchers are already
// validated: pointers non-NULL and aligned, 0 < M, N, 0 < K, K % 32 == 0,
// extents within the W4A16_MAX_* limits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4a16 {

constexpr int kGroup = 32;

// Decode/verify path: dequant-on-the-fly GEMV with activations held in VGPRs.
hipError_t launch_gemv(const float *X, const int32_t *qweight, const float *scales, float *Y,
                       int M, int N, int K, hipStream_t stream);

// The kernel launch_gemv runs for an M x N x K shape (one of W4A16_GEMV_*).
int gemv_kernel(int M, int N, int K);

// Decode GEMV (M <= 8, any K) on the 4x4x4 fp16 matrix instructions:
// exact weight codes, two fp16 limbs of each group-prescaled activation.
// launch_gemv runs it whenever gemv_mfma_supported(M, K).
bool gemv_mfma_supported(int M, int K);
int gemv_mfma_quads(int N);
hipError_t launch_gemv_mfma(const float *X, const int32_t *qweight, const float *scales, float *Y,
                            int M, int N, int K, hipStream_t stream);
// the same with the fused gate/up SwiGLU epilogue (W: 2F rows, gate then up; Y[M][F])
hipError_t launch_gemv_mfma_swiglu(const float *X, const int32_t *qweight, const float *scales,
                                   float *Y, int M, int F, int K, hipStream_t stream);
// The same kernel on the weights of w4a16_repack (bit for bit its result on
// the public layout).
hipError_t launch_gemv_mfma_packed(const float *X, const void *packed, float *Y, int M, int N,
                                   int K, hipStream_t stream);

// Skinny GEMM (any M >= 1) on the fp16 matrix instructions: exact weight
// codes, two fp16 limbs of each activation prescaled per row and pair of
// groups, fp32 accumulation; no workspace.  Up to kSkinnyAlwaysM rows it is
// always the matrix-core choice; above, skinny_preferred(M, N) compares its
// rounds of workgroups with the 128 x 128 tile's.
constexpr int kSkinnyAlwaysM = 64;
bool skinny_supported(int M);
bool skinny_preferred(int M, int N);
hipError_t launch_skinny(const float *X, const int32_t *qweight, const float *scales, float *Y,
                         int M, int N, int K, hipStream_t stream);
// the skinny kernel with the fused gate/up SwiGLU epilogue (W: 2F rows, gate
// then up; Y[M][F])
hipError_t launch_skinny_swiglu(const float *X, const int32_t *qweight, const float *scales,
                                float *Y, int M, int F, int K, hipStream_t stream);
// the skinny kernel on w4a16_repack's layout (one expert of the grouped pack)
hipError_t launch_skinny_repacked(const float *X, const void *packed, float *Y, int M, int N,
                                  int K, hipStream_t stream);

// Tiled path: fp32 MFMA (32x32x2) on weight tiles dequantized into registers.
hipError_t launch_tile(const float *X, const int32_t *qweight, const float *scales, float *Y,
                       int M, int N, int K, hipStream_t stream);
// Large-M matrix-core tile: fp16 MFMA on exact weight codes and two fp16 limbs
// of each activation (prescaled per row and pair of groups inside the kernel);
// 128 x 128 tiles, no workspace.
long tile_mx_tiles(int M, int N);
hipError_t launch_tile_mx(const float *X, const int32_t *qweight, const float *scales, float *Y,
                          int M, int N, int K, hipStream_t stream);
// the same kernel on the layout w4a16_repack writes (one expert of the grouped layout)
hipError_t launch_tile_mx_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                                 hipStream_t stream);

// Split-precision path: fp16 MFMA on exact weight codes and two fp16 limbs of
// each activation; needs a caller workspace of split_workspace_bytes(M, N, K).
size_t split_workspace_bytes(int M, int N, int K);
hipError_t launch_split(const float *X, const int32_t *qweight, const float *scales, float *Y,
                        int M, int N, int K, void *workspace, hipStream_t stream);
// Packed weights for the split path (one-time repack of qweight and scales
// into the kernel's stage layout) and the GEMM on them.
size_t split_pack_bytes(int N, int K);
hipError_t launch_split_pack(const int32_t *qweight, const float *scales, void *packed, int N,
                             int K, hipStream_t stream);
hipError_t launch_split_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                               void *workspace, hipStream_t stream);
// The split path with the tile (64 x 16 J WN), the K split S and the pipeline
// depth D fixed by the caller instead of chosen by the library's plan;
// `weights` is qweight (scales separate) or, with `packed`, a packed buffer.
size_t split_workspace_bytes_with(int M, int N, int K, int J, int WN, int S);
hipError_t launch_split_with(const float *X, const void *weights, const float *scales, bool packed,
                             float *Y, int M, int N, int K, int J, int WN, int S, int D,
                             void *workspace, hipStream_t stream);

// Fused gate/up SwiGLU on the GEMV path: W has 2F rows (gate, then up);
// Y[M][F] = silu(X . gate^T) * (X . up^T).
hipError_t launch_gemv_swiglu(const float *X, const int32_t *qweight, const float *scales,
                              float *Y, int M, int F, int K, hipStream_t stream);

// Grouped (MoE) GEMM: Y[r] = X[token_index[r]] . dequant(W_e)^T for the
// expert e whose slot range [offsets[e], offsets[e+1]) holds r.
// which kernel launch_grouped runs for this shape: 1 matrix cores, 2 fp32
// FMA with staged token rows, 3 fp32 FMA reading activations from memory
int grouped_kernel(int T, int R, int E, int N, int K);

// small-M GEMM (1 <= M <= 64) on weights packed by the grouped repack (one
// expert); workspace: the split-K partials (0 bytes when K is not split)
bool small_packed_supported(int M);
size_t small_packed_workspace_bytes(int M, int N, int K);
hipError_t launch_small_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                               void *workspace, hipStream_t stream);
// The allocation-free form's scratch: a file-scope device array of
// kNoAllocScratchBytes per device; noalloc_scratch gives its device address
// on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);
// the packed layout of the grouped path: bytes, repack, the packed GEMM and
// whether a shape can use it
size_t grouped_pack_bytes(int E, int N, int K);
hipError_t launch_grouped_pack(const int32_t *qweight, const float *scales, void *packed, int E,
                               int N, int K, hipStream_t stream);
bool grouped_packed_supported(int T, int R, int E, int N, int K);
hipError_t launch_grouped_packed(const float *X, const int32_t *token_index,
                                 const int32_t *offsets, const void *packed, float *Y, int T,
                                 int R, int E, int N, int K, hipStream_t stream);
hipError_t launch_grouped(const float *X, const int32_t *token_index, const int32_t *offsets,
                          const int32_t *qweight, const float *scales, float *Y, int T, int R,
                          int E, int N, int K, hipStream_t stream);

// the fp32 FMA GEMV kernels whatever M and K (the matrix-core GEMV is not
// considered)
hipError_t launch_gemv_fma(const float *X, const int32_t *qweight, const float *scales, float *Y,
                           int M, int N, int K, hipStream_t stream);

// Measurement helper: one launch streaming n <= 4 device segments (16-byte
// aligned, byte counts multiples of 16) with `loads` 16-byte loads per thread
// and `threads` threads per block; sink receives at most one word.
hipError_t launch_read_floor(const void *const *ptrs, const long *bytes, int n, int threads,
                             int loads, unsigned *sink, hipStream_t stream);


}  // namespace w4a16
