// Device helpers shared by the GEMV-style kernels (gemv.hip, grouped.hip):
// streaming loads of one 16-byte group of W and of its scale, the group dot
// product with the weights as exact signed bytes 16*(q - 8), and DPP sums
// over aligned lane segments.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float load_stream4(const float *p) { return __builtin_nontemporal_load(p); }

// SwiGLU epilogue of the fused gate/up GEMV: silu(g) * u, silu(g) = g / (1 + exp(-g))
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// sum over the group of x_k * 16*(q_k - 8): the 16*(q-8) are exact signed
// bytes, each met by one fp32 FMA (one rounding per term).
__device__ __forceinline__ float group_dot16(const float (&x)[32], uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte b of hi: high nibble of byte b (k = 8j+2b+1) in bits 4..7, sign bit flipped
    const uint32_t hi = (u[j] & 0xF0F0F0F0u) ^ 0x80808080u;
    // byte b of lo: low nibble of byte b (k = 8j+2b) moved to bits 4..7, sign bit flipped
    const uint32_t lo = ((u[j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a0 = fmaf(x[8 * j + 2 * b], float(int8_t(lo >> (8 * b))), a0);
      a1 = fmaf(x[8 * j + 2 * b + 1], float(int8_t(hi >> (8 * b))), a1);
    }
  }
  return a0 + a1;
}

// The same for MT activation rows at once: each weight is converted once and
// met by the MT rows' activations (MT FMAs per weight instead of MT
// conversions and MT FMAs).
template <int MT>
__device__ __forceinline__ void group_dot16_rows(const float (&x)[MT][32], uint4 w,
                                                 float (&out)[MT]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float a0[MT], a1[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) a0[m] = a1[m] = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t hi = (u[j] & 0xF0F0F0F0u) ^ 0x80808080u;
    const uint32_t lo = ((u[j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float fl = float(int8_t(lo >> (8 * b)));
      const float fh = float(int8_t(hi >> (8 * b)));
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        a0[m] = fmaf(x[m][8 * j + 2 * b], fl, a0[m]);
        a1[m] = fmaf(x[m][8 * j + 2 * b + 1], fh, a1[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) out[m] = a0[m] + a1[m];
}

// Sum over aligned segments of Z lanes (Z = 16, 32 or 64); the last lane of
// each segment receives the segment total.  Row shifts 1, 2, 4, 8 accumulate
// each 16-lane row into its lane 15 (lanes past the row edge read 0),
// row_bcast:15 adds lane 15 of rows 0 and 2 into rows 1 and 3, and
// row_bcast:31 adds lane 31 into rows 2 and 3.
template <int Z>
__device__ __forceinline__ float segment_sum(float v) {
  static_assert(Z == 16 || Z == 32 || Z == 64, "segment of 16, 32 or 64 lanes");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  if constexpr (Z >= 32)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  if constexpr (Z >= 64)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}

}  // namespace
}  // namespace w4a16
