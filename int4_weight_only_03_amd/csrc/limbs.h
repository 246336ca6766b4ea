// Device helpers of the fp16 matrix-core kernels (split, grouped, decode GEMV,
// skinny and large-M tiles): the power-of-two prescale and two-limb split of
// fp32 activations, and the conversion of packed nibbles to exact fp16 weight
// codes (q - 8).
//
// Each activation row is scaled by 2^e so that its largest magnitude lies in
// [2^14, 2^15), then split into hi = f16(x'), lo = f16(x' - hi), whose sum
// holds x' to 22 significant bits; every product of a limb and a code is
// exact in fp32.  Within each 8-wide block of k the limbs are laid out in the
// order the nibble conversion produces: x0 x4 x1 x5 x2 x6 x3 x7.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace w4a16 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// exponent e with max|x| * 2^e in [2^14, 2^15); 0 for a zero or non-finite max
__device__ __forceinline__ int row_exponent(float mx) {
  int e = 0;
  if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
    int E;
    frexpf(mx, &E);  // mx in [2^(E-1), 2^E)
    e = 15 - E;
  }
  return e;
}

__device__ __forceinline__ void split_block(const float4 a, const float4 c, int e, half8_t &h,
                                            half8_t &l) {
  const float v[8] = {a.x, c.x, a.y, c.y, a.z, c.z, a.w, c.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xs = ldexpf(v[i], e);
    const _Float16 hv = (_Float16)xs;
    h[i] = hv;
    l[i] = (_Float16)(xs - (float)hv);
  }
}

// f16 (q - 8) pairs from one word of 8 nibbles: VGPR p holds nibbles p, p+4.
// (w & mask) | 0x6400 puts a nibble into the mantissa of 1024 (v_bitop3).
__device__ __forceinline__ half8_t nibbles_to_f16(uint32_t w) {
  const uint32_t t = w >> 8;
  const half2_t p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64006400u, 0xEA));
  const half2_t p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64006400u, 0xEA));
  const half2_t p2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(t, 0x000F000Fu, 0x64006400u, 0xEA));
  const half2_t p3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(t, 0x00F000F0u, 0x64006400u, 0xEA));
  const half2_t c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const half2_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t r0 = p0 - c1032;       // (1024 + q) - 1032
  const half2_t r1 = p1 * c16 - c72;   // (1024 + 16q) / 16 - 72
  const half2_t r2 = p2 - c1032;
  const half2_t r3 = p3 * c16 - c72;
  half8_t o;
  o[0] = r0[0]; o[1] = r0[1]; o[2] = r1[0]; o[3] = r1[1];
  o[4] = r2[0]; o[5] = r2[1]; o[6] = r3[0]; o[7] = r3[1];
  return o;
}

// max(|a|, |b|, |c|) in one instruction (fmaxf on loaded values costs a
// canonicalising max per operand).  IEEE maxNum: a quiet NaN operand is
// passed over.
__device__ __forceinline__ float limb_absmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Limbs of two prescaled activations t0 = x0 2^(e+11), t1 = x1 2^(e+11) as
// fp16 pairs (t0 in the low half): hi = f16(t 2^-11), lo = f16(t - 2^11 hi),
// one mixed-precision FMA each, both rounded to nearest.  k = 2^-11, m = -2^11.
__device__ __forceinline__ void limb_split2(float t0, float t1, float k, float m, uint32_t &hi,
                                          uint32_t &lo) {
  asm("v_fma_mixlo_f16 %0, %2, %4, 0\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0\n\t"
      "v_fma_mixlo_f16 %1, %0, %5, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %0, %5, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(hi), "=&v"(lo)
      : "v"(t0), "v"(t1), "v"(k), "v"(m));
}

}  // namespace
}  // namespace w4a16
