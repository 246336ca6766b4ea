// Decode GEMV (M <= 8) on the 4x4x4 fp16 matrix instructions.
//
// The decode path exists for memory-bound MoE inference and aims at the HBM
// bandwidth peak ("The Quiet Commit: How a Single Plan Update Closed Phase 3
// of a Native DDTree Inference Engine", sections "Input and Output Knowledge"
// and "The Thinking Process"); unpacking must not eat the bandwidth that
// 4-bit storage saves ("The Silence of Success: A Single Line That Speaks
// Volumes", section "Assumptions Embedded in the Code").  On gfx950 an fp32
// FMA per weight plus its conversion left the kernel bound by VALU issue
// even with every operand in cache; here the products go to the matrix
// cores and the VALU only converts nibbles (about 1.1 operations per weight).
//
// Arithmetic (the split path's, per group instead of per row):
//  * Each group of 32 activations is scaled by 2^e so that its largest
//    magnitude lies in [2^14, 2^15) (e at most 116, so that 2^(e+11) is a
//    normal fp32 number; only groups below 2^-101 are scaled less), and split
//    into fp16 limbs hi = f16(x'), lo = f16((x' - hi) * 2^11), from
//    t = x * 2^(e+11) with one mixed-precision FMA each; x' = hi + 2^-11 lo
//    to 22 significant bits for every activation down to 2^-28 of the group
//    maximum, and to an absolute 2^-50 of that maximum below it (lo carries
//    2^11 so that it stays out of the fp16 subnormals).  Products of a limb
//    and an exact fp16 weight code (q - 8) are exact in fp32.
//  * v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products.  Block b
//    of a wave is group g = 16*wave + b.  Its A operand (4 x 4) holds the limb
//    rows (hi and lo of two activation rows; M = 3..8 take up to four A
//    operands against the same converted weights), its B operand (4 x 4) four W
//    rows; eight instructions cover the group's 32 k, accumulating from zero.
//    Lane 4b + j is W row j as B operand and receives D[.][j] (the limb sums
//    of that row), so the lane that loaded a row's 16 bytes and scale also
//    applies the scale: y += (s * 2^-e) * (D_hi + 2^-11 D_lo), one group at a time,
//    so no group ever mixes with another's scale.
//  * Sums over groups: 4-lane strides inside 16-lane rows by DPP rotation,
//    across the wave's rows by permlane swaps, across waves in LDS in wave
//    order.  No atomics: every output is summed in a fixed order.
//
// Fused gate/up SwiGLU (kSw): W holds 2F rows, gate rows 0..F-1 then up rows
// F..2F-1.  A workgroup's 4R outputs n need gate row n and up row F + n, so a
// lane carries 2R row quads (gate quads, then up quads); the writer stores
// silu(gate) * up and neither product reaches memory.
//
// Loads: each lane first loads its 8 activations (the group's quarter j) and
// then all of its weight and scale loads, so the weights stream while the
// activations are split.  All are buffer loads whose resources end at the
// last valid byte (the activation row at K, the workgroup's weights and
// scales at row N): rows past N and groups past K read zero, with no clamped
// addresses or selects, and each load's address is one 32-bit offset.  One
// workgroup covers 4R rows and all groups (one wave per 16 groups up to
// K = 8192; beyond, 16 waves taking blocks of 16 groups in turn, one pass of
// loads, split and products per block), about one workgroup per compute
// unit.

#include "w4a16_internal.h"
#include "gemv_common.h"
#include "limbs.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

constexpr int kMxMaxWaves = 16;   // one pass of 16 groups each: K <= 8192
constexpr int kMxLongWaves = 8;   // longer K: passes of 8 blocks of 16 groups (256 VGPRs a wave)
// word 3 of a raw buffer resource (32-bit data format, no swizzle)
constexpr int kRsrcWord3 = 0x00020000;

// LDS: per wave [16 groups][limb rows of one A operand][4 quarters] of 8 fp16:
// 2 limb rows for MT = 1 (2 KB), 4 otherwise (4 KB); with MT > 2 the A
// operands pass through it one after the other.  Once a wave has read its
// limbs back, the start of its region holds its [MT][4*RL] partial sums.
constexpr int mx_limb_rows(int MT) { return MT == 1 ? 2 : 4; }
constexpr size_t mx_wave_lds(int MT) { return size_t(16) * mx_limb_rows(MT) * 64; }
static_assert(mx_wave_lds(1) >= 1 * 4 * 8 * sizeof(float), "partials fit the limb region");
static_assert(mx_wave_lds(8) >= 8 * 4 * 4 * sizeof(float), "partials fit the limb region");
// (row quads per lane: at most 8 for MT <= 2, 4 for MT = 4, 2 for MT = 8)

// One workgroup: rows rowbase .. rowbase + 4R - 1 of the N x K matrix at
// qw/sc (kSw: gate rows there, up rows N further) against MT activation rows
// xr[m] (rows past the real ones point at a real row and feed only results
// that are not stored), results to yr[m][n] for yr[m] != nullptr and n < N.
//
// kPk: W in the repacked layout of w4a16_repack instead (qw its weight
// blocks, sc its scales, S4 steps of 4 groups per 16-row tile, T16 tiles):
// each lane gathers the same 16 bytes (words 0..3 of its group and row) from
// four chunks 256 bytes apart, so the arithmetic and its result are those of
// the public layout, bit for bit.
template <int MT, int R, bool kSw, bool kPk, bool kLong>
__device__ __forceinline__ void mx_pass(const float *const (&xr)[MT], const uint4 *__restrict__ qw,
                                        const float *__restrict__ sc, float *const (&yr)[MT],
                                        int N, int G, long rowbase, unsigned char *smem, int S4,
                                        long T16) {
  static_assert(!(kSw && kPk), "the fused SwiGLU reads the public layout only");
  constexpr int RL = kSw ? 2 * R : R;  // row quads per lane (gate quads, then up quads)
  constexpr int MS = (MT + 1) / 2;     // A operands of 4 limb rows (2 activation rows each)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int b = lane >> 2, j = lane & 3;
  // kLong (K beyond 16 waves of 16 groups): the waves take blocks of 16
  // groups in turn, block wave + nw * it in pass it, each pass's sums adding
  // into acc; otherwise one pass.
  const int nw = int(blockDim.x >> 6);
  const int passes = kLong ? (G + 16 * nw - 1) / (16 * nw) : 1;
  float acc[MT][RL];
  for (int it = 0; it < passes; ++it) {
  const int g = (wave + nw * it) * 16 + b;
  const bool gv = g < G;

  // Buffer loads: a workgroup's weight rows start its buffers, which end at
  // row N (or at its last row), so rows past N read zero; a lane past the last
  // group (g >= G) reads zero too (its offsets lie past every buffer).  The
  // activation rows' buffers end at K: those lanes' activations are zero.
  const uint32_t K4 = uint32_t(G) * kGroup * 4;
  u32x4 xw[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(xr[m]), (short)0, int(K4), kRsrcWord3);
    const uint32_t vx = uint32_t(g) * (kGroup * 4) + 32u * uint32_t(j);
    xw[m][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, vx, 0, 0);
    xw[m][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, vx + 16, 0, 0);
  }
  uint4 w[RL];
  float s[RL];
  if constexpr (kPk) {
    // the workgroup's rows lie in tiles t0 .. t0 + 1 (4R <= 32 rows, rowbase a
    // multiple of 4R); the buffers end at the last tile, so rows past it read
    // zero, and the tiles' padding rows and groups hold weight 0, scale 0
    const long t0 = rowbase >> 4;
    const long t1 = std::min((rowbase + 4 * R + 15) >> 4, T16);
    const int bytes = int(t1 - t0) * S4 * 1024;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4 *>(qw + t0 * S4 * 64), (short)0, bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(sc + t0 * S4 * 64), (short)0, bytes / 4, kRsrcWord3);
    const bool in = g < 4 * S4;  // past the padded groups: offsets past the buffers
    const int st = g >> 2, gq = g & 3;
#pragma unroll
    for (int q = 0; q < RL; ++q) {
      const int rl = int(rowbase & 15) + 4 * q + j;  // row within tile t0 (and t0 + 1)
      const int blk = (rl >> 4) * S4 + st;
      const uint32_t ow = in ? uint32_t(((blk * 64 + (rl & 15)) * 16) + gq * 4) : 0x40000000u;
      const uint32_t os = in ? uint32_t(((blk * 16 + (rl & 15)) * 4 + gq) * 4) : 0x40000000u;
      w[q].x = __builtin_amdgcn_raw_buffer_load_b32(rw, ow, 0, 2);
      w[q].y = __builtin_amdgcn_raw_buffer_load_b32(rw, ow + 256, 0, 2);
      w[q].z = __builtin_amdgcn_raw_buffer_load_b32(rw, ow + 512, 0, 2);
      w[q].w = __builtin_amdgcn_raw_buffer_load_b32(rw, ow + 768, 0, 2);
      s[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 2));
    }
  } else {
    const int rows = int(std::min(long(N) - rowbase, long(4 * R)));
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4 *>(qw + rowbase * G), (short)0, rows * G * 16, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(sc + rowbase * G), (short)0, rows * G * 4, kRsrcWord3);
    __amdgpu_buffer_rsrc_t rwu = rw, rsu = rs;
    if constexpr (kSw) {
      rwu = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4 *>(qw + (long(N) + rowbase) * G),
                                              (short)0, rows * G * 16, kRsrcWord3);
      rsu = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(sc + (long(N) + rowbase) * G),
                                              (short)0, rows * G * 4, kRsrcWord3);
    }
    const uint32_t e0 = gv ? uint32_t(j * G + g) : 0x08000000u;  // element offset of row j
#pragma unroll
    for (int q = 0; q < RL; ++q) {
      const uint32_t eq = e0 + uint32_t(4 * (q % R) * G);
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(q >= R ? rwu : rw, eq * 16, 0, 2);
      w[q] = make_uint4(v.x, v.y, v.z, v.w);
      s[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(q >= R ? rsu : rs, eq * 4, 0, 2));
    }
  }

  // group maxima (the 4 lanes of a quad hold one group), exponents, limbs;
  // A operand p holds limb rows 4p .. 4p+3 (activation rows 2p, 2p+1), staged
  // through the wave's own LDS region (LDS operations of one wave complete in
  // order, so each read sees the writes before it and precedes the writes
  // after it).  With MT = 1, rows 2 and 3 repeat rows 0 and 1; the products of
  // a row depend only on that row, and those D rows are unused.
  constexpr int LR = mx_limb_rows(MT);
  half8_t *lb = reinterpret_cast<half8_t *>(smem + wave * mx_wave_lds(MT));
  float inv[MT];
  half8_t a[MS][4];
#pragma unroll
  for (int p = 0; p < MS; ++p) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int m = 2 * p + hh;
      if (m >= MT) break;
      const float v[8] = {__uint_as_float(xw[m][0].x), __uint_as_float(xw[m][0].y),
                          __uint_as_float(xw[m][0].z), __uint_as_float(xw[m][0].w),
                          __uint_as_float(xw[m][1].x), __uint_as_float(xw[m][1].y),
                          __uint_as_float(xw[m][1].z), __uint_as_float(xw[m][1].w)};
      // the group's largest magnitude (a NaN is passed over and still turns
      // the row's products to NaN)
      const float t0 = limb_absmax3(v[0], v[1], v[2]);
      const float t1 = limb_absmax3(v[3], v[4], v[5]);
      float mx = limb_absmax3(v[6], v[7], t0);
      mx = limb_absmax3(mx, t1, 0.0f);
      mx = limb_absmax3(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0xB1, 0xf, 0xf, false)), 0.0f);
      mx = limb_absmax3(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xf, 0xf, false)), 0.0f);
      // e in [-113, 116]: 2^-e and 2^(e+11) are normal, x * 2^(e+11) exact
      const int e = std::min(row_exponent(mx), 116);
      inv[m] = __int_as_float((127 - e) << 23);
      const float up = __int_as_float((127 + e + 11) << 23);
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) limb_split2(v[i] * up, v[4 + i] * up, 0x1p-11f, -2048.0f, hw[i], lw[i]);
      lb[(b * LR + 2 * hh) * 4 + j] = __builtin_bit_cast(half8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      lb[(b * LR + 2 * hh + 1) * 4 + j] = __builtin_bit_cast(half8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c) a[p][c] = lb[(b * LR + (MT == 1 ? (j & 1) : j)) * 4 + c];
    if (p + 1 < MS) __builtin_amdgcn_wave_barrier();  // the next operand's writes stay behind
  }

#pragma unroll
  for (int q = 0; q < RL; ++q) {
    const uint32_t u[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
    floatx4 d[MS];
#pragma unroll
    for (int p = 0; p < MS; ++p) d[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // word c: k = 8c..8c+7 in the order of split_block
      const half8_t bw = nibbles_to_f16(u[c]);
      const half4_t b0 = {bw[0], bw[1], bw[2], bw[3]};
      const half4_t b1 = {bw[4], bw[5], bw[6], bw[7]};
#pragma unroll
      for (int p = 0; p < MS; ++p) {  // independent accumulators: the MFMAs interleave
        const half4_t a0 = {a[p][c][0], a[p][c][1], a[p][c][2], a[p][c][3]};
        const half4_t a1 = {a[p][c][4], a[p][c][5], a[p][c][6], a[p][c][7]};
        d[p] = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d[p], 0, 0, 0);
        d[p] = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d[p], 0, 0, 0);
      }
    }
#pragma unroll
    for (int p = 0; p < MS; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = 2 * p + h;
        if (m < MT) {
          const float sp = s[q] * inv[m];  // exact: a power-of-two factor
          const float v = sp * fmaf(d[p][2 * h + 1], 0x1p-11f, d[p][2 * h]);
          acc[m][q] = it == 0 ? v : acc[m][q] + v;
        }
      }
  }
  }  // passes

  // sum over the wave's groups: lanes with equal j
  float *red = reinterpret_cast<float *>(smem + wave * mx_wave_lds(MT));  // this wave's own region
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < RL; ++q) {
      float v = acc[m][q];
      v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror:4
      v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror:8
      const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = __uint_as_float(h32[0]) + __uint_as_float(h32[1]);
      const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = __uint_as_float(h16[0]) + __uint_as_float(h16[1]);
      if (lane < 4) red[m * (4 * RL) + 4 * q + lane] = v;
    }
  __syncthreads();
  for (int o = threadIdx.x; o < MT * 4 * R; o += blockDim.x) {
    const int m = o / (4 * R), r = o - m * (4 * R);
    float v = 0.0f, u = 0.0f;
    for (int ww = 0; ww < int(blockDim.x >> 6); ++ww) {
      const float *p = reinterpret_cast<const float *>(smem + ww * mx_wave_lds(MT)) + m * (4 * RL);
      v += p[r];
      if (kSw) u += p[4 * R + r];
    }
    const long n = rowbase + r;
    if (yr[m] != nullptr && n < N) yr[m][n] = kSw ? silu_mul(v, u) : v;
  }
}

// N: outputs per row of Y (F for kSw, whose W has 2N rows).  MT = 4 serves
// M = 3 and 4, MT = 8 serves M = 5 .. 8.
template <int MT, int R, bool kSw, bool kPk, bool kLong>
__global__ void __launch_bounds__(kLong ? 64 * kMxLongWaves : 64 * kMxMaxWaves)
gemv_mx(const float *__restrict__ X, const uint4 *__restrict__ qw, const float *__restrict__ sc,
        float *__restrict__ Y, int M, int N, int G, int S4, long T16) {
  extern __shared__ __align__(16) unsigned char smem[];
  const long K = long(G) * kGroup;
  const float *xr[MT];
  float *yr[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    xr[m] = X + (m < M ? m : 0) * K;
    yr[m] = m < M ? Y + long(m) * N : nullptr;
  }
  mx_pass<MT, R, kSw, kPk, kLong>(xr, qw, sc, yr, N, G, long(blockIdx.x) * (4 * R), smem, S4, T16);
}

template <int MT, int R, bool kSw, bool kPk>
hipError_t run_mx(const float *X, const void *qw, const float *sc, float *Y, int M, int N,
                  int G, hipStream_t stream) {
  const bool lng = G > 16 * kMxMaxWaves;
  const int waves = lng ? kMxLongWaves : (G + 15) / 16;
  const int blocks = int((long(N) + 4 * R - 1) / (4 * R));
  const int S4 = (G + 3) / 4;
  const long T16 = (long(N) + 15) / 16;
  if (lng)
    hipLaunchKernelGGL((gemv_mx<MT, R, kSw, kPk, true>), dim3(blocks), dim3(waves * 64),
                       waves * mx_wave_lds(MT), stream, X, reinterpret_cast<const uint4 *>(qw), sc,
                       Y, M, N, G, S4, T16);
  else
    hipLaunchKernelGGL((gemv_mx<MT, R, kSw, kPk, false>), dim3(blocks), dim3(waves * 64),
                       waves * mx_wave_lds(MT), stream, X, reinterpret_cast<const uint4 *>(qw), sc,
                       Y, M, N, G, S4, T16);
  return hipGetLastError();
}

template <int MT, bool kSw, bool kPk = false>
hipError_t dispatch_mx(int R, const float *X, const void *qw, const float *sc, float *Y, int M,
                       int N, int G, hipStream_t stream) {
  // row quads per lane are capped so that no variant spills: 8 only for the
  // plain GEMV of up to 2 rows, 2 (1 with kSw) for 8 rows
  constexpr int kCap = MT <= 2 ? (kSw ? 4 : 8) : (MT == 4 ? 4 : (kSw ? 1 : 2));
  R = std::min(R, kCap);
  switch (R) {
    case 8:
      if constexpr (kCap >= 8) return run_mx<MT, 8, kSw, kPk>(X, qw, sc, Y, M, N, G, stream);
      else return hipErrorInvalidValue;
    case 4:
      if constexpr (kCap >= 4) return run_mx<MT, 4, kSw, kPk>(X, qw, sc, Y, M, N, G, stream);
      else return hipErrorInvalidValue;
    case 2:
      if constexpr (kCap >= 2) return run_mx<MT, 2, kSw, kPk>(X, qw, sc, Y, M, N, G, stream);
      else return hipErrorInvalidValue;
    default: return run_mx<MT, 1, kSw, kPk>(X, qw, sc, Y, M, N, G, stream);
  }
}

}  // namespace

bool gemv_mfma_supported(int M, int K) {
  return M >= 1 && M <= 8 && K >= kGroup;
}

// Quads of rows per lane: the most that still leaves at least 224 workgroups
// (most of the 256 compute units busy), at least one.
int gemv_mfma_quads(int N) {
  int R = 1;
  for (int r : {8, 4, 2})
    if ((long(N) + 4 * r - 1) / (4 * r) >= 224) {
      R = r;
      break;
    }
  return R;
}

hipError_t launch_gemv_mfma(const float *X, const int32_t *qweight, const float *scales, float *Y,
                            int M, int N, int K, hipStream_t stream) {
  if (!gemv_mfma_supported(M, K)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int R = gemv_mfma_quads(N);
  switch (M) {
    case 1: return dispatch_mx<1, false>(R, X, qweight, scales, Y, M, N, G, stream);
    case 2: return dispatch_mx<2, false>(R, X, qweight, scales, Y, M, N, G, stream);
    case 3:
    case 4: return dispatch_mx<4, false>(R, X, qweight, scales, Y, M, N, G, stream);
    default: return dispatch_mx<8, false>(R, X, qweight, scales, Y, M, N, G, stream);
  }
}

hipError_t launch_gemv_mfma_swiglu(const float *X, const int32_t *qweight, const float *scales,
                                   float *Y, int M, int F, int K, hipStream_t stream) {
  if (!gemv_mfma_supported(M, K)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int R = std::min(gemv_mfma_quads(F), 4);  // each lane carries gate and up quads
  switch (M) {
    case 1: return dispatch_mx<1, true>(R, X, qweight, scales, Y, M, F, G, stream);
    case 2: return dispatch_mx<2, true>(R, X, qweight, scales, Y, M, F, G, stream);
    case 3:
    case 4: return dispatch_mx<4, true>(R, X, qweight, scales, Y, M, F, G, stream);
    default: return dispatch_mx<8, true>(R, X, qweight, scales, Y, M, F, G, stream);
  }
}

hipError_t launch_gemv_mfma_packed(const float *X, const void *packed, float *Y, int M, int N,
                                   int K, hipStream_t stream) {
  if (!gemv_mfma_supported(M, K)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int R = gemv_mfma_quads(N);
  // the scales follow the T16 * S4 kilobyte weight blocks
  const float *psc = reinterpret_cast<const float *>(
      static_cast<const unsigned char *>(packed) + ((long(N) + 15) / 16) * ((G + 3) / 4) * 1024);
  switch (M) {
    case 1: return dispatch_mx<1, false, true>(R, X, packed, psc, Y, M, N, G, stream);
    case 2: return dispatch_mx<2, false, true>(R, X, packed, psc, Y, M, N, G, stream);
    case 3:
    case 4: return dispatch_mx<4, false, true>(R, X, packed, psc, Y, M, N, G, stream);
    default: return dispatch_mx<8, false, true>(R, X, packed, psc, Y, M, N, G, stream);
  }
}

}  // namespace w4a16
