// Skinny W4A16 GEMM on the fp16 matrix cores: Y[M][N] = X[M][K] . dequant(W)^T
// for a few dozen to a few hundred rows of X, with no workspace.
//
// The pages' speculative decoder scores a tree of draft tokens in one batch
// against every weight ("The Quiet Commit: How a Single Documentation Edit
// Marks the Completion of a Major Engineering Milestone", section "The
// Context: A Native DDTree Engine Takes Shape"): M of a few dozen rows, too
// many for a GEMV and too few to reuse a weight tile in fp32 matrix
// instructions at their peak.  This kernel is w4a16_gemm's path for
// 9 <= M <= 64 (and for 3 <= M <= 8 when K is beyond the decode GEMV's limit),
// and above 64 rows while its rounds of workgroups cost less than those of the
// 128 x 128 matrix-core tile (skinny_preferred).
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
#define W4A16_SK_WAVES 8
#endif
#ifndef W4A16_SK_P
#define W4A16_SK_P 1
#endif
constexpr int kSkWaves = W4A16_SK_WAVES;  // waves per workgroup, splitting the K range
constexpr int kSkP = W4A16_SK_P;          // steps in flight per wave (LDS slots)
constexpr int kSkSG = 4;                  // groups per step
// one slot: the step's activations (16*MT rows x 512 B), weight words (16*NT
// W rows x 64 B) and scales (16*NT W rows x 16 B)
__host__ __device__ constexpr int sk_xbytes(int MT) { return 16 * MT * kSkSG * 128; }
__host__ __device__ constexpr int sk_slot(int MT, int NT) {
  return sk_xbytes(MT) + NT * 16 * kSkSG * 16 + NT * 16 * kSkSG * 4;
}

typedef __attribute__((address_space(3))) void sk_lds_void;

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

// An empty asm that claims to change x: keeps a loop-invariant offset's
// uses (and their zero extension) inside the loop.
__device__ __forceinline__ void sk_opaque(uint32_t &x) { asm volatile("" : "+v"(x)); }

// kSw: fused gate/up SwiGLU (public layout): W holds 2N rows, gate rows
// 0..N-1 then up rows N..2N-1; a workgroup's first NT/2 column tiles are gate
// rows and its last NT/2 the up rows of the same outputs, and the store
// writes silu(gate) * up.
template <int MT, int NT, int P, bool kRP, bool kSw = false>
__global__ void __launch_bounds__(64 * kSkWaves)
skinny_mx(const float *__restrict__ X, const uint32_t *__restrict__ qw,
          const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G,
          int tiles_n) {
  constexpr int SG = kSkSG;
  constexpr int kSlot = sk_slot(MT, NT);
  static_assert(P >= 1 && P <= 2, "ring depth");
  // Each ring entry's slots and the row factors are LDS objects of their
  // own, so that the compiler can tell a read of one from the direct copies
  // into another (else it waits for every copy in flight before any LDS
  // read, the row factors' included).
  __shared__ __align__(16) unsigned char sk_ring0[kSkWaves * kSlot];
  __shared__ __align__(16) unsigned char sk_ring1[P > 1 ? kSkWaves * kSlot : 16];
  __shared__ __align__(16) float sk_finv[kSkWaves * 16 * MT];
  constexpr int kRows = 16 * MT;         // rows of X staged per wave
  constexpr int kRowBytes = SG * 128;    // one row of one step: 32 chunks of 16 bytes
  constexpr int kCopies = kRows * kRowBytes / 1024;  // 1 KB activation copies per step
  constexpr int kWOff = sk_xbytes(MT);               // weight words in the slot
  constexpr int kSOff = kWOff + NT * 1024;           // scales in the slot
  // VMEM operations per step: the activation copies, NT weight copies, NT
  // scale copies
  constexpr int kStepOps = kCopies + 2 * NT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int c = lane & 15, R = lane >> 4;
  const int nb = blockIdx.x % tiles_n, mb = blockIdx.x / tiles_n;
  static_assert(!kSw || (!kRP && NT % 2 == 0), "SwiGLU: public layout, gate and up tiles");
  constexpr int NO = kSw ? NT / 2 : NT;  // output column tiles
  const int m0 = mb * 16 * MT, n0 = nb * 16 * NO;
  const int S = G / SG;  // whole steps
  const int s0 = int(long(S) * wave / kSkWaves), s1 = int(long(S) * (wave + 1) / kSkWaves);
  // this wave's staging slot of ring entry v
  auto slot_of = [&](int v) -> unsigned char * {
    return (v == 0 ? sk_ring0 : sk_ring1) + wave * kSlot;
  };
  float *finv = sk_finv + wave * kRows;

  // Activation copies: copy j, lane i writes LDS bytes 16 i .. 16 i + 15 of
  // the slot's kilobyte j: staged row rho = 2 j + i / 32, physical chunk
  // p = i % 32, which holds the row's logical chunk p ^ (rho & 15) (an XOR
  // swizzle: the 16 rows an operand read touches at one logical chunk fall in
  // 16 distinct chunks of one 256-byte window, hence distinct LDS banks).
  // Rows past M read row M-1.  Every copy's address is a wave-uniform base
  // (the tile's first row, the step's first group) plus a fixed per-lane byte
  // offset below 2^23 (16 rows of at most 2^17 floats).
  uint32_t xoff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int rho = 2 * j + lane / 32;
    const int L = (lane & 31) ^ (rho & 15);
    xoff[j] = uint32_t(std::min(m0 + rho, M - 1) - m0) * uint32_t(G) * 128u + 16u * uint32_t(L);
  }
  // Weight copy t: lane i writes 16 bytes at slot offset 1024 t + 16 i: W row
  // n0 + 16 t + i / 4, position i % 4 of that row's 64 bytes, which holds
  // group (i % 4 - i / 16) % 4 of the step (each row's groups rotated by
  // row / 4, so that the 16 rows a read touches at one group fall in distinct
  // banks).  Scale copy t: lane i writes 4 bytes at offset 256 t + 4 i of the
  // scales: the scale of group i % 4 of the same row.  Rows past N read row
  // N-1.  Offsets relative to the tile's first row (below 2^23 bytes).
  const int wg = ((lane & 3) - (lane >> 4)) & 3;  // group of this lane's weight copy
  uint32_t woff[NT], soff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int to = t % NO;  // the output tile (kSw: gate tiles, then up tiles)
    const uint32_t wrow = uint32_t(std::min(n0 + 16 * to + lane / 4, N - 1) - n0);
    woff[t] = (wrow * uint32_t(G) + uint32_t(wg)) * 16u;
    soff[t] = (wrow * uint32_t(G) + uint32_t(lane & 3)) * 4u;
  }
  const char *wtile = reinterpret_cast<const char *>(qw) + long(n0) * G * 16;
  const char *stile = reinterpret_cast<const char *>(sc) + long(n0) * G * 4;
  // kSw: the up rows sit N rows further
  const char *wtile_u = wtile + (kSw ? long(N) * G * 16 : 0);
  const char *stile_u = stile + (kSw ? long(N) * G * 4 : 0);
  // kRP: qw is w4a16_repack's buffer, a 1 KB block per (16-row tile, 4-group
  // step) with lane l's 16 bytes its operand words for the 4 groups (word
  // l / 16 of each, row l % 16), then a 256-byte block of the 16 rows' 4
  // scales; the padding (rows to 16, groups to 4) holds weight and scale 0.
  // Tiles past the last read the last one (never stored).
  const int T16 = (N + 15) / 16, S4 = (G + SG - 1) / SG;
  const char *pw = reinterpret_cast<const char *>(qw);
  const char *ps = pw + long(T16) * S4 * 1024;
  int ptile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ptile[t] = std::min(n0 / 16 + t, T16 - 1);

  // Step s's copies into slot v (kTail: the step past the whole steps, whose
  // groups past G re-read group G-1, masked later).  The offsets pass
  // through an empty asm so that their zero extension stays beside the
  // copies, which then take the scalar-base form.
  auto load = [&](int v, int s, auto kTail) {
    constexpr bool tail = decltype(kTail)::value;
    unsigned char *slot = slot_of(v);
    const long gs = long(s) * SG;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) sk_opaque(xoff[j]);
    if constexpr (!kRP) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sk_opaque(woff[t]);
        sk_opaque(soff[t]);
      }
    } else {
      // whole blocks of the repacked buffer, the partial last step included
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const long blk = long(ptile[t]) * S4 + s;
        const char *wsrc = pw + blk * 1024 + 16 * lane;
        __builtin_amdgcn_global_load_lds(wsrc, (sk_lds_void *)(slot + kWOff + 1024 * t), 16, 0, 0);
        const char *ssrc = ps + blk * 256 + 4 * lane;
        __builtin_amdgcn_global_load_lds(ssrc, (sk_lds_void *)(slot + kSOff + 256 * t), 4, 0, 0);
      }
    }
    if (!tail) {
      const char *xb = reinterpret_cast<const char *>(X) + long(m0) * G * 128 + gs * 128;
#pragma unroll
      for (int j = 0; j < kCopies; ++j) {
        const char *src = xb + xoff[j];
        __builtin_amdgcn_global_load_lds(src, (sk_lds_void *)(slot + 1024 * j), 16, 0, 0);
      }
      if constexpr (!kRP) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const char *wsrc = (t < NO ? wtile : wtile_u) + gs * 16 + woff[t];
          __builtin_amdgcn_global_load_lds(wsrc, (sk_lds_void *)(slot + kWOff + 1024 * t), 16, 0,
                                           0);
          const char *ssrc = (t < NO ? stile : stile_u) + gs * 4 + soff[t];
          __builtin_amdgcn_global_load_lds(ssrc, (sk_lds_void *)(slot + kSOff + 256 * t), 4, 0, 0);
        }
      }
    } else {
      const char *xb = reinterpret_cast<const char *>(X) + long(m0) * G * 128;
#pragma unroll
      for (int j = 0; j < kCopies; ++j) {
        const int rho = 2 * j + lane / 32;
        const uint32_t q = uint32_t(((lane & 31) ^ (rho & 15)) >> 3);  // the chunk's group
        const char *src =
            xb + std::min(gs + q, long(G) - 1) * 128 + (xoff[j] - 128u * q);
        __builtin_amdgcn_global_load_lds(src, (sk_lds_void *)(slot + 1024 * j), 16, 0, 0);
      }
      if constexpr (!kRP) {
        const long gw = std::min(gs + wg, long(G) - 1);
        const long gsc = std::min(gs + (lane & 3), long(G) - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const char *wsrc = (t < NO ? wtile : wtile_u) + gw * 16 + (woff[t] - 16u * uint32_t(wg));
          __builtin_amdgcn_global_load_lds(wsrc, (sk_lds_void *)(slot + kWOff + 1024 * t), 16, 0,
                                           0);
          const char *ssrc =
              (t < NO ? stile : stile_u) + gsc * 4 + (soff[t] - 4u * uint32_t(lane & 3));
          __builtin_amdgcn_global_load_lds(ssrc, (sk_lds_void *)(slot + kSOff + 256 * t), 4, 0, 0);
        }
      }
    }
  };

  // A step's operands, copied from its slot into registers (after which the
  // slot can take the next copies): this lane's activations of row 16u + c,
  // group g, k = 8R .. 8R+7 (logical chunks 8g + 2R and 8g + 2R + 1), word R
  // of group g of W row 16t + c, and that row's scales of the step's groups.
  struct Ops {
    float4 x[MT][SG][2];
    uint32_t w[NT][SG];
    float4 sc[NT];
  };
  auto fetch = [&](int v, Ops &o) {
    const unsigned char *slot = slot_of(v);
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
      for (int g = 0; g < SG; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pch = (8 * g + 2 * R + h) ^ c;  // (16u + c) & 15 == c
          o.x[u][g][h] =
              *reinterpret_cast<const float4 *>(slot + (16 * u + c) * kRowBytes + 16 * pch);
        }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (kRP) {
        const uint4 w4 = *reinterpret_cast<const uint4 *>(slot + kWOff + 1024 * t + 16 * lane);
        o.w[t][0] = w4.x;
        o.w[t][1] = w4.y;
        o.w[t][2] = w4.z;
        o.w[t][3] = w4.w;
      } else {
#pragma unroll
        for (int g = 0; g < SG; ++g)
          o.w[t][g] = *reinterpret_cast<const uint32_t *>(slot + kWOff + 1024 * t + 64 * c +
                                                          16 * ((g + (c >> 2)) & 3) + 4 * R);
      }
      o.sc[t] = *reinterpret_cast<const float4 *>(slot + kSOff + 256 * t + 16 * c);
    }
  };

  float acc[MT][NT][4];
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][t][r] = 0.0f;

  // one step, in two pairs of groups (one power of two per row and pair);
  // kMask for the step past the whole steps, whose groups past G count as
  // zero
  auto process = [&](int s, const Ops &o, auto kMask) {
    constexpr bool mask = decltype(kMask)::value;
    const int gb = s * SG;
#pragma unroll
    for (int pr = 0; pr < SG / 2; ++pr) {
      float4 xv[MT][2][2];
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            xv[u][q][h] = (!mask || gb + 2 * pr + q < G) ? o.x[u][2 * pr + q][h]
                                                         : make_float4(0.f, 0.f, 0.f, 0.f);
      // the pair's largest magnitude per row: a tree of three-operand
      // maxima over this lane's 16 values, then over the row's 4 lanes
      // (a NaN is passed over here and still turns the row's products to NaN)
      int e[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const float4 a0 = xv[u][0][0], a1 = xv[u][0][1], a2 = xv[u][1][0], a3 = xv[u][1][1];
        const float t0 = limb_absmax3(a0.x, a0.y, a0.z);
        const float t1 = limb_absmax3(a0.w, a1.x, a1.y);
        const float t2 = limb_absmax3(a1.z, a1.w, a2.x);
        const float t3 = limb_absmax3(a2.y, a2.z, a2.w);
        const float t4 = limb_absmax3(a3.x, a3.y, a3.z);
        const float t5 = limb_absmax3(t0, t1, a3.w);
        float mx = limb_absmax3(t2, t3, t4);
        mx = limb_absmax3(mx, t5, 0.0f);
        const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = limb_absmax3(__uint_as_float(h32[0]), __uint_as_float(h32[1]), 0.0f);
        const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = limb_absmax3(__uint_as_float(h16[0]), __uint_as_float(h16[1]), 0.0f);
        // e in [-113, 116]: 2^-e and 2^(e+11) are normal fp32 numbers.  A
        // row whose pair maximum lies below 2^-102 keeps fewer limb bits; its
        // absolute error stays below 2^-120 of the weights' magnitude.
        e[u] = std::min(row_exponent(mx), 116);
        if (R == 0) finv[16 * u + c] = __int_as_float((127 - e[u]) << 23);
      }
      // 2^(e+11) per row: x * 2^(e+11) is exact and finite (|x| 2^e < 2^15)
      float up[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) up[u] = ldexpf(1.0f, e[u] + 11);
      // the factors of this lane's result rows 4R .. 4R+3 (this wave's own
      // LDS words: its LDS operations complete in order)
      float4 fac[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u)
        fac[u] = *reinterpret_cast<const float4 *>(finv + 16 * u + 4 * R);

      float ss[MT][NT][4];  // the pair's sum, group scales applied, 2^-e not yet
      const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int g = 2 * pr + q;
        half8_t hi[MT], lo[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          // t = x 2^(e+11) (exact); hi = f16(t 2^-11); lo = f16(t - 2^11 hi),
          // the difference exact in fp32; order x0 x4 x1 x5 x2 x6 x3 x7
          const float4 a = xv[u][q][0], b4 = xv[u][q][1];
          const float va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {b4.x, b4.y, b4.z, b4.w};
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            limb_split2(va[i] * up[u], vb[i] * up[u], 0x1p-11f, -2048.0f, hw[i], lw[i]);
          hi[u] = __builtin_bit_cast(half8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
          lo[u] = __builtin_bit_cast(half8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const half8_t b = nibbles_to_f16(o.w[t][g]);
          const _Float16 k2 = (_Float16)0x1p-11f;
          const half8_t b2 = b * half8_t{k2, k2, k2, k2, k2, k2, k2, k2};  // exact in fp16
          const float s4[4] = {o.sc[t].x, o.sc[t].y, o.sc[t].z, o.sc[t].w};
          const float sq = (!mask || gb + g < G) ? s4[g] : 0.0f;
#pragma unroll
          for (int u = 0; u < MT; ++u) {
            floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[u], b, zero, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[u], b2, d, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              ss[u][t][r] = q == 0 ? sq * d[r] : fmaf(sq, d[r], ss[u][t][r]);
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
    }
  };

  // The ring: slot v holds the steps s with (s - s0) % P == v.  Per step:
  // wait until only the later slots' operations are in flight; move the
  // slot's operands into registers; once those reads are done, start the
  // slot's copies of step s + P; then do the arithmetic, under the copies.
  // (A wave's last reloads repeat its last step: never used, they keep the
  // number of operations in flight the same for every step.)
  const std::false_type whole;
  if (s0 < s1) {
#pragma unroll
    for (int v = 0; v < P; ++v) load(v, std::min(s0 + v, s1 - 1), whole);
  }
  int s = s0;
  for (; s + P <= s1; s += P) {
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
      load(v, std::min(s + v + P, s1 - 1), whole);
      // the reload stays ahead of the step's arithmetic
      __builtin_amdgcn_sched_barrier(0);
      process(s + v, o, whole);
    }
  }
  asm volatile("" ::: "memory");
  sk_wait_vm<0>();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int v = 0; v < P - 1; ++v)
    if (s + v < s1) {
      Ops o;
      fetch(v, o);
      process(s + v, o, whole);
    }
  // the groups past the whole steps (G % 4 of them), on the last wave, from
  // slot 0 (free: every copy of this wave is done and read)
  if (G % SG != 0 && wave == kSkWaves - 1) {
    const std::true_type tail;
    asm volatile("" ::: "memory");
    sk_wait_lgkm0();
    asm volatile("" ::: "memory");
    load(0, S, tail);
    asm volatile("" ::: "memory");
    sk_wait_vm<0>();
    asm volatile("" ::: "memory");
    Ops o;
    fetch(0, o);
    process(S, o, tail);
  }

  // the waves' partial tiles, added in wave order (the slots are free once
  // every wave is past its loop)
  constexpr int kTile = MT * NT * 4 * 64;
  static_assert(kTile * 4 <= kSlot, "partials fit the first ring entry");
  float *red = reinterpret_cast<float *>(sk_ring0);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave * kTile + ((u * NT + t) * 4 + r) * 64 + lane] = acc[u][t][r];
  __syncthreads();
  if constexpr (kSw) {
    // gate tile t and up tile t + NO hold the same outputs
    for (int i = threadIdx.x; i < MT * NO * 256; i += 64 * kSkWaves) {
      const int l = i & 63, r = (i >> 6) & 3, ut = i >> 8;
      const int u = ut / NO, t = ut - u * NO;
      const int ig = ((u * NT + t) * 4 + r) * 64 + l, iu = ig + NO * 256;
      float g = 0.0f, v = 0.0f;
#pragma unroll
      for (int w = 0; w < kSkWaves; ++w) {
        g += red[w * kTile + ig];
        v += red[w * kTile + iu];
      }
      const int m = m0 + 16 * u + 4 * (l >> 4) + r;
      const int n = n0 + 16 * t + (l & 15);
      if (m < M && n < N) Y[long(m) * N + n] = silu_mul(g, v);
    }
  } else {
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
  p.tiles_m = int((long(M) + 15) / 16);
  p.NT = 1;
  for (int nt = 4; nt > 1; nt /= 2)
    if ((long(N) + 16 * nt - 1) / (16 * nt) * p.tiles_m >= 256) {
      p.NT = nt;
      break;
    }
#endif
  p.tiles_n = int((long(N) + 16 * p.NT - 1) / (16 * p.NT));
  return p;
}

template <int MT, int NT, bool kRP>
hipError_t run_skinny(const SkPlan &p, const float *X, const void *qw, const float *sc,
                      float *Y, int M, int N, int G, hipStream_t stream) {
  const long blocks = long(p.tiles_m) * p.tiles_n;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((skinny_mx<MT, NT, kSkP, kRP>), dim3(unsigned(blocks)), dim3(64 * kSkWaves),
                     0, stream, X, reinterpret_cast<const uint32_t *>(qw), sc, Y, M, N, G,
                     p.tiles_n);
  return hipGetLastError();
}

template <bool kRP>
hipError_t dispatch_skinny(const float *X, const void *qw, const float *sc, float *Y, int M,
                           int N, int K, hipStream_t stream) {
  if (!skinny_supported(M)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const SkPlan p = plan_skinny(M, N);
#ifdef W4A16_SK_MT
  if (p.MT == 2)
    return p.NT == 1 ? run_skinny<2, 1, kRP>(p, X, qw, sc, Y, M, N, G, stream)
                     : run_skinny<2, 2, kRP>(p, X, qw, sc, Y, M, N, G, stream);
#endif
  return p.NT == 1   ? run_skinny<1, 1, kRP>(p, X, qw, sc, Y, M, N, G, stream)
         : p.NT == 2 ? run_skinny<1, 2, kRP>(p, X, qw, sc, Y, M, N, G, stream)
                     : run_skinny<1, 4, kRP>(p, X, qw, sc, Y, M, N, G, stream);
}

}  // namespace

bool skinny_supported(int M) { return M >= 1; }

// Rounds of workgroups over the 256 compute units, weighted by the work of
// one: a skinny workgroup of 16 x 16 NT outputs costs NT units, a 128 x 128
// matrix-core tile 33 (per round, both in proportion to K: 24.2 us for a round
// of 16 x 64 skinny tiles and 200 us for a round of 128 x 128 tiles at
// K = 7168, measured on MI355X).  Below the crossover the tile's rounds are
// mostly idle compute units (one workgroup per unit for all of K).
bool skinny_preferred(int M, int N) {
  if (M <= kSkinnyAlwaysM) return true;
  const SkPlan p = plan_skinny(M, N);
  const long sk_rounds = (long(p.tiles_m) * p.tiles_n + 255) / 256;
  const long tile_rounds = (tile_mx_tiles(M, N) + 255) / 256;
  return sk_rounds * p.NT <= tile_rounds * 33;
}

hipError_t launch_skinny(const float *X, const int32_t *qweight, const float *scales, float *Y,
                         int M, int N, int K, hipStream_t stream) {
  return dispatch_skinny<false>(X, qweight, scales, Y, M, N, K, stream);
}

hipError_t launch_skinny_repacked(const float *X, const void *packed, float *Y, int M, int N,
                                  int K, hipStream_t stream) {
  return dispatch_skinny<true>(X, packed, nullptr, Y, M, N, K, stream);
}

// The fused SwiGLU form: W has 2F rows; workgroups of 16 rows of X by 16 NT/2
// outputs (NT = 4 when that leaves at least 256 workgroups, else 2).
hipError_t launch_skinny_swiglu(const float *X, const int32_t *qweight, const float *scales,
                                float *Y, int M, int F, int K, hipStream_t stream) {
  if (!skinny_supported(M)) return hipErrorInvalidValue;
  const int G = K / kGroup;
  SkPlan p;
  p.MT = 1;
  p.tiles_m = int((long(M) + 15) / 16);
  p.NT = (long(F) + 31) / 32 * p.tiles_m >= 256 ? 4 : 2;
  p.tiles_n = int((long(F) + 8 * p.NT - 1) / (8 * p.NT));
  const long blocks = long(p.tiles_m) * p.tiles_n;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (p.NT == 4)
    hipLaunchKernelGGL((skinny_mx<1, 4, kSkP, false, true>), dim3(unsigned(blocks)),
                       dim3(64 * kSkWaves), 0, stream, X,
                       reinterpret_cast<const uint32_t *>(qweight), scales, Y, M, F, G, p.tiles_n);
  else
    hipLaunchKernelGGL((skinny_mx<1, 2, kSkP, false, true>), dim3(unsigned(blocks)),
                       dim3(64 * kSkWaves), 0, stream, X,
                       reinterpret_cast<const uint32_t *>(qweight), scales, Y, M, F, G, p.tiles_n);
  return hipGetLastError();
}

}  // namespace w4a16
