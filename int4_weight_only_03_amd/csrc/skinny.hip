// Skinny W4A16 GEMM on the fp16 matrix cores: Y[M][N] = X[M][K] . dequant(W)^T
// for a few dozen rows of X, with no workspace.
//
// The pages' speculative decoder scores a tree of draft tokens in one batch
// against every weight ("The Quiet Commit: How a Single Documentation Edit
// Marks the Completion of a Major Engineering Milestone", section "The
// Context: A Native DDTree Engine Takes Shape"): M of a few dozen rows, too
// many for a GEMV and too few to reuse a weight tile in fp32 matrix
// instructions at their peak.  This kernel is w4a16_gemm's path for
// 9 <= M <= 64 (and for 3 <= M <= 8 when K is beyond the decode GEMV's limit).
//
// Arithmetic: the decode GEMV's (exact weight codes, two fp16 limbs of each
// prescaled activation, fp32 accumulation), with the power of two taken per
// row of X and step of SG = 2 groups: the step's largest magnitude goes into
// [2^14, 2^15), hi = f16(x * 2^e), lo = f16((x * 2^e - hi) * 2^11).  Every
// activation down to 2^-28 of its step maximum keeps 22 significant bits.  The
// low limb meets the weight codes times 2^-11 (exact in fp16), so both limbs'
// products land in one fp32 accumulator: d = sum hi*(q-8) + sum lo*(q-8)*2^-11.
// Each group's d takes its scale with one FMA into the step sum; each step sum
// takes 2^-e with one FMA into the running total.
//
// Mapping: v_mfma_f32_16x16x32_f16, A = activation limbs (16 rows of X), B =
// weight codes (16 rows of W).  Lane (c, R) (c = lane % 16, R = lane / 16)
// holds the A operand of row c, k = 8R .. 8R+7 of the group, the B operand of
// W row c, word R of the group, and the result D[4R + r][c], r = 0..3: its
// column n = c is the W row whose scale it loaded.  The 4 lanes of a row
// (equal c) hold its 32 k of the group; the row maximum over a step is taken
// across them with permlane swaps, and the factors 2^-e reach the result
// layout (rows 4R + r) through the wave's own LDS words.
//
// Workgroup: a tile of 16*MT rows of X by 16*NT rows of W; its waves split
// the K range in steps.  Each step's activations, weight words and scales
// reach the wave's LDS slots by direct copies (global_load_lds); the wave
// moves a step's operands into registers, starts the copies of a later step
// into the freed slot, and only then does the step's arithmetic, so the
// copies run under it.  The waves' partial tiles are added in wave order in
// LDS (deterministic, no atomics).

#include "w4a16_internal.h"
#include "gemv_common.h"
#include "limbs.h"

#include <algorithm>
#include <type_traits>

namespace w4a16 {
namespace {

#ifndef W4A16_SK_WAVES
#define W4A16_SK_WAVES 16
#endif
#ifndef W4A16_SK_P
#define W4A16_SK_P 1
#endif
constexpr int kSkWaves = W4A16_SK_WAVES;  // waves per workgroup, splitting the K range
constexpr int kSkSG = 2;         // groups per step (one power of two per row and step)
constexpr int kSkP = W4A16_SK_P;  // steps in flight per wave (LDS slots)
// one slot: the step's activations (16*MT rows x 256 B), weight words (32 W
// rows x 32 B) and scales (32 W rows x 8 B)
__host__ __device__ constexpr int sk_xbytes(int MT) { return 16 * MT * kSkSG * 128; }
// weight and scale copies per step: one per 32 rows of W (at least one)
__host__ __device__ constexpr int sk_wcopies(int NT) { return NT < 2 ? 1 : NT / 2; }
__host__ __device__ constexpr int sk_wbytes(int NT) { return sk_wcopies(NT) * 32 * kSkSG * 16; }
__host__ __device__ constexpr int sk_sbytes(int NT) { return sk_wcopies(NT) * 32 * kSkSG * 4; }
__host__ __device__ constexpr int sk_slot(int MT, int NT) {
  return sk_xbytes(MT) + sk_wbytes(NT) + sk_sbytes(NT);
}

typedef __attribute__((address_space(3))) void sk_lds_void;

// LDS: per wave kSkP slots and 16*MT row factors; the partial tiles of the
// final reduction reuse the slots
__host__ __device__ constexpr int sk_lds_bytes(int MT, int NT) {
  return kSkWaves * (kSkP * sk_slot(MT, NT) + 16 * MT * 4);
}

// s_waitcnt with vmcnt = VM (lgkmcnt, expcnt not waited for)
template <int VM>
__device__ __forceinline__ void sk_wait_vm() {
  static_assert(VM >= 0 && VM < 64, "wait count");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x70 | (15 << 8));
}
// s_waitcnt lgkmcnt(0) (vmcnt, expcnt not waited for)
__device__ __forceinline__ void sk_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | 0x70);
}

// max(|a|, |b|, |c|) in one instruction (fmaxf on loaded values costs a
// canonicalising max per operand).  IEEE maxNum: a quiet NaN operand is
// passed over.
__device__ __forceinline__ float sk_absmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// An empty asm that claims to change x: keeps a loop-invariant offset's
// uses (and their zero extension) inside the loop.
__device__ __forceinline__ void sk_opaque(uint32_t &x) { asm volatile("" : "+v"(x)); }

// Limbs of two prescaled activations t0 = x0 2^(e+11), t1 = x1 2^(e+11) as
// fp16 pairs (t0 in the low half): hi = f16(t 2^-11), lo = f16(t - 2^11 hi),
// one mixed-precision FMA each, both rounded to nearest.  k = 2^-11, m = -2^11.
__device__ __forceinline__ void sk_split2(float t0, float t1, float k, float m, uint32_t &hi,
                                          uint32_t &lo) {
  asm("v_fma_mixlo_f16 %0, %2, %4, 0\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0\n\t"
      "v_fma_mixlo_f16 %1, %0, %5, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %0, %5, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(hi), "=&v"(lo)
      : "v"(t0), "v"(t1), "v"(k), "v"(m));
}

template <int MT, int NT, int SG, int P>
__global__ void __launch_bounds__(64 * kSkWaves)
skinny_mx(const float *__restrict__ X, const uint32_t *__restrict__ qw,
          const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G,
          int tiles_n) {
  extern __shared__ __align__(16) unsigned char sk_lds[];
  constexpr int kRows = 16 * MT;                 // rows of X staged per wave
  constexpr int kRowBytes = SG * 128;            // one row of one step
  constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per staged row
  constexpr int kCopies = kRows * kRowBytes / 1024;  // 1 KB activation copies per step
  constexpr int kSlot = sk_slot(MT, NT);
  constexpr int kWC = sk_wcopies(NT);
  static_assert(SG == kSkSG && kChunks == 16, "a staged row is 16 chunks");
  // VMEM operations per step: the activation copies, one weight copy, one
  // scale copy
  constexpr int kStepOps = kCopies + 2 * kWC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int c = lane & 15, R = lane >> 4;
  const int nb = blockIdx.x % tiles_n, mb = blockIdx.x / tiles_n;
  const int m0 = mb * 16 * MT, n0 = nb * 16 * NT;
  const long K = long(G) * kGroup;
  const int S = (G + SG - 1) / SG;  // steps
  const int s0 = int(long(S) * wave / kSkWaves), s1 = int(long(S) * (wave + 1) / kSkWaves);
  unsigned char *slots = sk_lds + wave * (P * kSlot);             // this wave's staging slots
  float *finv = reinterpret_cast<float *>(sk_lds + kSkWaves * P * kSlot) + wave * kRows;

  // Activation copies: copy j, lane i writes LDS bytes 16 i .. 16 i + 15 of
  // the slot's kilobyte j: staged row rho = 4 j + i / 16, physical chunk
  // p = i % 16, which holds the row's logical chunk p ^ (rho & 15) (an XOR
  // swizzle: the 16 rows an operand read touches at one logical chunk fall in
  // 16 distinct chunks, hence distinct LDS banks; each lane quad still reads
  // 64 contiguous bytes).  Rows past M read row M-1.  Every copy's address is
  // a wave-uniform base (the step's first group) plus a fixed per-lane byte
  // offset below 2^32 (X holds at most 64 rows of 2^17 floats).
  uint32_t xoff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int rho = 4 * j + lane / 16;
    const int xchunk = (lane & 15) ^ (rho & 15);
    xoff[j] = uint32_t(std::min(m0 + rho, M - 1)) * uint32_t(K * 4) +
              uint32_t(128 * (xchunk >> 3) + 16 * (xchunk & 7));
  }
  // Weight copy jw: lane i writes the 16 bytes of group (i & 1) of the step
  // of W row n0 + 32 jw + i / 2 (rows past N read row N-1).  Scale copy jw:
  // lane i writes the scale of group (i & 1) of the same row.  Offsets
  // relative to the tile's first row (below 2^23 bytes).
  uint32_t woff[kWC], soff[kWC];
#pragma unroll
  for (int jw = 0; jw < kWC; ++jw) {
    const uint32_t wrow = uint32_t(std::min(n0 + 32 * jw + lane / 2, N - 1) - n0);
    woff[jw] = (wrow * uint32_t(G) + uint32_t(lane & 1)) * 16u;
    soff[jw] = (wrow * uint32_t(G) + uint32_t(lane & 1)) * 4u;
  }
  const char *wtile = reinterpret_cast<const char *>(qw) + long(n0) * G * 16;
  const char *stile = reinterpret_cast<const char *>(sc) + long(n0) * G * 4;

  // Step s's copies.  Only the last step of an odd G reaches past the end of
  // a row: there the second group's chunks re-read group G-1 (masked).
  auto load = [&](int v, int s) {
    unsigned char *slot = slots + v * kSlot;
    const long gs = long(s) * SG;
    // (the offsets pass through an empty asm so that their zero extension
    // stays beside the loads, which then take the scalar-base form)
#pragma unroll
    for (int j = 0; j < kCopies; ++j) sk_opaque(xoff[j]);
#pragma unroll
    for (int jw = 0; jw < kWC; ++jw) {
      sk_opaque(woff[jw]);
      sk_opaque(soff[jw]);
    }
    if (SG * (s + 1) <= G) {
      const char *xb = reinterpret_cast<const char *>(X) + gs * 128;
#pragma unroll
      for (int j = 0; j < kCopies; ++j) {
        const char *src = xb + xoff[j];
        __builtin_amdgcn_global_load_lds(src, (sk_lds_void *)(slot + j * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int jw = 0; jw < kWC; ++jw) {
        const char *wsrc = wtile + gs * 16 + woff[jw];
        __builtin_amdgcn_global_load_lds(wsrc, (sk_lds_void *)(slot + sk_xbytes(MT) + 1024 * jw),
                                         16, 0, 0);
        const char *ssrc = stile + gs * 4 + soff[jw];
        __builtin_amdgcn_global_load_lds(
            ssrc, (sk_lds_void *)(slot + sk_xbytes(MT) + sk_wbytes(NT) + 256 * jw), 4, 0, 0);
      }
    } else {
      const char *xb = reinterpret_cast<const char *>(X) + (G - 1) * 128L;
#pragma unroll
      for (int j = 0; j < kCopies; ++j) {
        const uint32_t q = uint32_t(((lane & 15) ^ ((4 * j + lane / 16) & 15)) >> 3);
        const char *src = xb + (xoff[j] - 128u * q);
        __builtin_amdgcn_global_load_lds(src, (sk_lds_void *)(slot + j * 1024), 16, 0, 0);
      }
      const uint32_t odd = uint32_t(lane & 1);
#pragma unroll
      for (int jw = 0; jw < kWC; ++jw) {
        const char *wsrc = wtile + (G - 1) * 16L + (woff[jw] - 16u * odd);
        __builtin_amdgcn_global_load_lds(wsrc, (sk_lds_void *)(slot + sk_xbytes(MT) + 1024 * jw),
                                         16, 0, 0);
        const char *ssrc = stile + (G - 1) * 4L + (soff[jw] - 4u * odd);
        __builtin_amdgcn_global_load_lds(
            ssrc, (sk_lds_void *)(slot + sk_xbytes(MT) + sk_wbytes(NT) + 256 * jw), 4, 0, 0);
      }
    }
  };

  float acc[MT][NT][4];
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][t][r] = 0.0f;

  // A step's operands, copied from its slot into registers (after which the
  // slot can take the next copies): this lane's activations of row 16u + c,
  // group q, k = 8R .. 8R+7 (logical chunks 8q + 2R and 8q + 2R + 1), word R
  // of group q of W row 16t + c and that row's scale of group q.
  struct Ops {
    float4 x[MT][SG][2];
    uint32_t w[NT][SG];
    float sc[NT][SG];
  };
  auto fetch = [&](int v, Ops &o) {
    const unsigned char *slot = slots + v * kSlot;
    const uint32_t *wst = reinterpret_cast<const uint32_t *>(slot + sk_xbytes(MT));
    const float *sst = reinterpret_cast<const float *>(slot + sk_xbytes(MT) + sk_wbytes(NT));
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int q = 0; q < SG; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rho = 16 * u + c;
          const int pch = (8 * q + 2 * R + h) ^ c;  // rho & 15 == c
          o.x[u][q][h] = *reinterpret_cast<const float4 *>(slot + rho * kRowBytes + 16 * pch);
        }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < SG; ++q) {
        o.w[t][q] = wst[((16 * t + c) * SG + q) * 4 + R];
        o.sc[t][q] = sst[(16 * t + c) * SG + q];
      }
  };

  // one step: kMask when some of its groups may lie past G (the last step
  // only), whose activations and scales then count as zero
  auto process = [&](int s, const Ops &o, auto kMask) {
    constexpr bool mask = decltype(kMask)::value;
    const int gb = s * SG;
    float4 xv[MT][SG][2];
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int q = 0; q < SG; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          xv[u][q][h] = (!mask || gb + q < G) ? o.x[u][q][h] : make_float4(0.f, 0.f, 0.f, 0.f);
    // the step's largest magnitude per row (fmaxf of magnitudes: a NaN is
    // passed over here and still turns the row's products to NaN), over this
    // lane's values, then over the row's 4 lanes
    int e[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      // a tree of three-operand maxima over the 4 SG values
      static_assert(SG == 2, "the maximum tree takes 16 values");
      float v16[16];
#pragma unroll
      for (int q = 0; q < SG; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 x4 = xv[u][q][h];
          v16[8 * q + 4 * h + 0] = x4.x;
          v16[8 * q + 4 * h + 1] = x4.y;
          v16[8 * q + 4 * h + 2] = x4.z;
          v16[8 * q + 4 * h + 3] = x4.w;
        }
      const float m0 = sk_absmax3(v16[0], v16[1], v16[2]);
      const float m1 = sk_absmax3(v16[3], v16[4], v16[5]);
      const float m2 = sk_absmax3(v16[6], v16[7], v16[8]);
      const float m3 = sk_absmax3(v16[9], v16[10], v16[11]);
      const float m4 = sk_absmax3(v16[12], v16[13], v16[14]);
      const float m5 = sk_absmax3(m0, m1, v16[15]);
      float mx = sk_absmax3(m2, m3, m4);
      mx = sk_absmax3(mx, m5, 0.0f);
      const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = sk_absmax3(__uint_as_float(h32[0]), __uint_as_float(h32[1]), 0.0f);
      const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = sk_absmax3(__uint_as_float(h16[0]), __uint_as_float(h16[1]), 0.0f);
      // e in [-113, 116]: 2^-e and 2^(e+11) are normal fp32 numbers.  A row
      // whose step maximum lies below 2^-102 keeps fewer limb bits; its
      // absolute error stays below 2^-120 of the weights' magnitude.
      e[u] = std::min(row_exponent(mx), 116);
      if (R == 0) finv[16 * u + c] = __int_as_float((127 - e[u]) << 23);
    }
    // 2^(e+11) per row: x * 2^(e+11) is exact and finite (|x| 2^e < 2^15)
    float up[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) up[u] = ldexpf(1.0f, e[u] + 11);
    // the factors of this lane's result rows 4R .. 4R+3 (this wave's own LDS
    // words: its LDS operations complete in order)
    float4 fac[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) fac[u] = *reinterpret_cast<const float4 *>(finv + 16 * u + 4 * R);

    float ss[MT][NT][4];  // the step's sum, group scales applied, 2^-e not yet
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss[u][t][r] = 0.0f;
    const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      half8_t hi[MT], lo[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        // t = x 2^(e+11) (exact); hi = f16(t 2^-11); lo = f16(t - 2^11 hi), the
        // difference exact in fp32; order x0 x4 x1 x5 x2 x6 x3 x7
        const float4 a = xv[u][q][0], b4 = xv[u][q][1];
        const float va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {b4.x, b4.y, b4.z, b4.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sk_split2(va[i] * up[u], vb[i] * up[u], 0x1p-11f, -2048.0f, hw[i], lw[i]);
        hi[u] = __builtin_bit_cast(half8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        lo[u] = __builtin_bit_cast(half8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const half8_t b = nibbles_to_f16(o.w[t][q]);
        const _Float16 k2 = (_Float16)0x1p-11f;
        const half8_t b2 = b * half8_t{k2, k2, k2, k2, k2, k2, k2, k2};  // exact in fp16
        const float sq = (!mask || gb + q < G) ? o.sc[t][q] : 0.0f;
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[u], b, zero, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[u], b2, d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) ss[u][t][r] = fmaf(sq, d[r], ss[u][t][r]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const float f[4] = {fac[u].x, fac[u].y, fac[u].z, fac[u].w};
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][t][r] = fmaf(ss[u][t][r], f[r], acc[u][t][r]);
    }
  };

  // The ring: slot v holds the steps s with (s - s0) % P == v.  Before a
  // slot's reads, wait until only the later slots' operations are in flight;
  // once its reads are done (its operands are in registers), reload it and
  // only then work on the operands, so that the copies overlap that work.
  if (s0 < s1) {
#pragma unroll
    for (int v = 0; v < P; ++v) load(v, std::min(s0 + v, s1 - 1));
  }
  // whole rings: none of their steps reaches past G (the last step of the K
  // range is always in the partial ring below, or the wave's last step)
  const int s_full = std::min(s1, S - 1);
  int s = s0;
  for (; s + P <= s_full; s += P) {
#pragma unroll
    for (int v = 0; v < P; ++v) {
      Ops o;
      asm volatile("" ::: "memory");
      sk_wait_vm<(P - 1) * kStepOps>();
      asm volatile("" ::: "memory");
      fetch(v, o);
      asm volatile("" ::: "memory");
      sk_wait_lgkm0();
      asm volatile("" ::: "memory");
      load(v, std::min(s + v + P, s1 - 1));
      // the reload stays ahead of the step's arithmetic
      __builtin_amdgcn_sched_barrier(0);
      process(s + v, o, std::false_type{});
    }
  }
  asm volatile("" ::: "memory");
  sk_wait_vm<0>();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int v = 0; v < P; ++v)
    if (s + v < s1) {
      Ops o;
      fetch(v, o);
      process(s + v, o, std::true_type{});
    }

  // the waves' partial tiles, added in wave order (the staging slots are free
  // once every wave is past its loop)
  constexpr int kTile = MT * NT * 4 * 64;
  static_assert(kTile * kSkWaves * 4 <= kSkWaves * kSkP * kSlot, "partials fit the slots");
  float *red = reinterpret_cast<float *>(sk_lds);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave * kTile + ((u * NT + t) * 4 + r) * 64 + lane] = acc[u][t][r];
  __syncthreads();
  for (int i = threadIdx.x; i < kTile; i += 64 * kSkWaves) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) v += red[w * kTile + i];
    const int l = i & 63, r = (i >> 6) & 3, ut = i >> 8;
    const int u = ut / NT, t = ut - u * NT;
    const int m = m0 + 16 * u + 4 * (l >> 4) + r;
    const int n = n0 + 16 * t + (l & 15);
    if (m < M && n < N) Y[long(m) * N + n] = v;
  }
}

struct SkPlan {
  int MT, NT, tiles_m, tiles_n;
};

// 16 rows of X per workgroup (each weight row is then read ceil(M / 16)
// times, each activation row ceil(N / (16 NT)) times); 64 or 32 rows of W when
// that still gives at least 256 workgroups (one per compute unit), else 16.
SkPlan plan_skinny(int M, int N) {
  SkPlan p;
#ifdef W4A16_SK_MT
  p.MT = W4A16_SK_MT;
  p.NT = W4A16_SK_NT;
  p.tiles_m = (M + 16 * p.MT - 1) / (16 * p.MT);
#else
  p.MT = 1;
  p.tiles_m = (M + 15) / 16;
  p.NT = 1;
  for (int nt = 4; nt > 1; nt /= 2)
    if (long((N + 16 * nt - 1) / (16 * nt)) * p.tiles_m >= 256) {
      p.NT = nt;
      break;
    }
#endif
  p.tiles_n = (N + 16 * p.NT - 1) / (16 * p.NT);
  return p;
}

template <int MT, int NT>
hipError_t run_skinny(const SkPlan &p, const float *X, const int32_t *qw, const float *sc,
                      float *Y, int M, int N, int G, hipStream_t stream) {
  const long blocks = long(p.tiles_m) * p.tiles_n;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((skinny_mx<MT, NT, kSkSG, kSkP>), dim3(unsigned(blocks)),
                     dim3(64 * kSkWaves), size_t(sk_lds_bytes(MT, NT)), stream,
                     X, reinterpret_cast<const uint32_t *>(qw), sc, Y, M, N, G, p.tiles_n);
  return hipGetLastError();
}

}  // namespace

bool skinny_supported(int M) { return M >= 1 && M <= kSkinnyMaxM; }

hipError_t launch_skinny(const float *X, const int32_t *qweight, const float *scales, float *Y,
                         int M, int N, int K, hipStream_t stream) {
  if (!skinny_supported(M)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const SkPlan p = plan_skinny(M, N);
#ifdef W4A16_SK_MT
  if (p.MT == 2)
    return p.NT == 1 ? run_skinny<2, 1>(p, X, qweight, scales, Y, M, N, G, stream)
                     : run_skinny<2, 2>(p, X, qweight, scales, Y, M, N, G, stream);
#endif
  return p.NT == 1   ? run_skinny<1, 1>(p, X, qweight, scales, Y, M, N, G, stream)
         : p.NT == 2 ? run_skinny<1, 2>(p, X, qweight, scales, Y, M, N, G, stream)
                     : run_skinny<1, 4>(p, X, qweight, scales, Y, M, N, G, stream);
}

}  // namespace w4a16
