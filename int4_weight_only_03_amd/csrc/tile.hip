// Tiled path of the W4A16 GEMM for larger M: Y = X . dequant(W)^T on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32).
//
// The pages' kernel accumulates in fp32 for fidelity ("The Silence of
// Success: A Single Line That Speaks Volumes", section "Assumptions Embedded
// in the Code") and its reference dequantizes first and then multiplies
// (same page, section "What the Edit Actually Built").  Here every weight is
// dequantized to exactly that fp32 value, fl32((nibble - 8) * scale), with one
// FMA (q*s + (-8s) rounded once), and the fp32 MFMA does the contraction.
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64): lane l supplies
// A[i = l%32][k = l/32] and B[k = l/32][j = l%32] and receives D[i][j] for
// j = l%32, i = 8*(r/4) + 4*(l/32) + r%4 in accumulator register r.
// For one group of 32 k, lane (l%32, h = l/32) owns the 16 k
// 32g + 8v + 4h + c (v, c = 0..3): four 16-byte loads of one X row at byte
// offsets 32v + 16h, so the two lanes of a row read 32 contiguous bytes per
// load (one 64-byte sector instead of two), and from one 16-byte load of the
// group's 4 words of one W row, nibbles 4h..4h+3 of each word.  The 16 MFMAs
// of the group each consume one (x, w) pair of the same k; any order of k
// within a group gives the same sum up to rounding.  Dequantization goes
// straight into the B registers: no LDS round trip, since the wave that
// dequantizes a weight is the wave that consumes it.
//
// A wave computes (32*WM) x (32*WN) outputs; a block has BWM x BWN such waves
// side by side and KS copies of that arrangement splitting the groups; the KS
// partial tiles are summed in LDS in a fixed order (deterministic, no atomics).
// The next group's raw loads are issued before the current group's MFMAs.
//
// Accumulation order.  The MFMAs of kAccGroups consecutive groups (16 each)
// accumulate from zero into block sums, and each block sum is added to the
// running total with one fp32 add.  A single chain over all of K would let
// the rounding error of sign-coherent products (every x*w >= 0) grow with the
// chain length until it leaves the tolerance near K = 2^17; with blocks of
// 8 groups the longest chain is 128 MFMAs plus K/256 block adds.  The skinny
// tiles split each block over CH = 2 independent chains (groups alternate
// between them), added to the total in chain order.
//
// Loads.  Each wave keeps a ring of P groups of raw operands in flight: the
// loop body is unrolled over the ring (slot u holds the groups with
// (g - g0) % P == u), each slot is reloaded right after its MFMAs, and the
// wait before a slot's MFMAs counts only the loads issued after its own.

#include "w4a16_internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kAccGroups = 8;  // groups per block sum (see "Accumulation order")
#ifndef W4A16_TILE_WIDE_PREFETCH
#define W4A16_TILE_WIDE_PREFETCH 2
#endif
#ifndef W4A16_TILE_SKINNY_PREFETCH
#define W4A16_TILE_SKINNY_PREFETCH 2
#endif
#ifndef W4A16_TILE_SKINNY_CHAINS
#define W4A16_TILE_SKINNY_CHAINS 2
#endif
#ifndef W4A16_TILE_SKINNY_SPLIT
#define W4A16_TILE_SKINNY_SPLIT 8
#endif
// groups of raw operands in flight per wave: 128 x 128 tiles, 32 x 32 tiles
constexpr int kWidePrefetch = W4A16_TILE_WIDE_PREFETCH;
constexpr int kSkinnyPrefetch = W4A16_TILE_SKINNY_PREFETCH;
constexpr int kSkinnyChains = W4A16_TILE_SKINNY_CHAINS;  // independent MFMA chains per wave
constexpr int kSkinnySplit = W4A16_TILE_SKINNY_SPLIT;    // waves splitting the groups

template <int WM, int WN, int BWM, int BWN, int KS, int P, int CH>
__global__ void __launch_bounds__(64 * BWM * BWN * KS)
tile_w4a16(const float *__restrict__ X, const uint32_t *__restrict__ qw,
           const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G,
           int tiles_n) {
  constexpr int BM = 32 * WM * BWM;
  constexpr int BN = 32 * WN * BWN;
  constexpr int WAVES_MN = BWM * BWN;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: kept in a scalar register, so
  // the group range and every loop branch below are scalar
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wk = wave / WAVES_MN;
  const int wmn = wave - wk * WAVES_MN;
  const int wm = wmn / BWN;
  const int wn = wmn - wm * BWN;
  const int bm = blockIdx.x / tiles_n;
  const int bn = blockIdx.x - bm * tiles_n;
  const int m_base = bm * BM + wm * 32 * WM;
  const int n_base = bn * BN + wn * 32 * WN;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const long K = long(G) * kGroup;
  const int g0 = int((long(G) * wk) / KS);
  const int g1 = int((long(G) * (wk + 1)) / KS);

  // Rows outside M / N read a valid row (their outputs are never stored).
  const float *xrow[WM];
#pragma unroll
  for (int a = 0; a < WM; ++a) {
    const int m = std::min(m_base + 32 * a + l32, M - 1);
    xrow[a] = X + long(m) * K + 4 * h;
  }
  const uint4 *qrow[WN];
  const float *srow[WN];
#pragma unroll
  for (int b = 0; b < WN; ++b) {
    const int n = std::min(n_base + 32 * b + l32, N - 1);
    qrow[b] = reinterpret_cast<const uint4 *>(qw + long(n) * (long(G) * 4));
    srow[b] = sc + long(n) * G;
  }
  const int nib_shift = 16 * h;  // nibbles 4h..4h+3 of each word

  // CH independent chains of MFMAs (group g feeds chain (g - g0) % CH), each
  // the block sum of its groups in the current block of kAccGroups groups
  static_assert(P % CH == 0 && kAccGroups % CH == 0, "chains follow the ring");
  floatx16 acc[CH][WM][WN];
  floatx16 tot[WM][WN];  // sum of the finished blocks
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        tot[a][b][r] = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c][a][b][r] = 0.0f;
      }

  // A ring of P groups of raw operands in flight.  Slot u always holds the
  // groups g with (g - g0) % P == u, so the loop body is unrolled P times and
  // no register is copied on the back edge; a load past the wave's range
  // re-reads its last group (always in bounds) and is never consumed.
  struct Slot {
    float4 xa[WM][4];
    uint4 wq[WN];
    float ws[WN];
  };
  Slot slot[P];
  auto load = [&](Slot &sl, int g) {
#pragma unroll
    for (int a = 0; a < WM; ++a) {
      const float4 *p = reinterpret_cast<const float4 *>(xrow[a] + long(g) * kGroup);
#pragma unroll
      for (int v = 0; v < 4; ++v) sl.xa[a][v] = p[2 * v];
    }
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      sl.wq[b] = qrow[b][g];
      sl.ws[b] = srow[b][g];
    }
  };
  auto consume = [&](const Slot &sl, floatx16 (&ac)[WM][WN]) {
    float wc[WN][16];
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const float s = sl.ws[b];
      const float neg8s = -8.0f * s;
      const uint32_t u[4] = {sl.wq[b].x, sl.wq[b].y, sl.wq[b].z, sl.wq[b].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // word v holds k = 8v .. 8v+7; this lane takes nibbles 4h .. 4h+3
        const uint32_t t = u[v] >> nib_shift;
        const uint32_t lo = t & 0x0F0Fu;         // nibbles 4h, 4h+2 in bytes 0, 1
        const uint32_t hi = (t >> 4) & 0x0F0Fu;  // nibbles 4h+1, 4h+3
        const float q[4] = {float(lo & 0xFFu), float(hi & 0xFFu), float(lo >> 8),
                            float(hi >> 8)};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          // (q - 8) * s rounded once: q*s - 8s is exact before the FMA's rounding
          wc[b][4 * v + c] = fmaf(q[c], s, neg8s);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) {
          const float4 &x4 = sl.xa[a][i >> 2];
          const float xv = (i & 3) == 0 ? x4.x : (i & 3) == 1 ? x4.y : (i & 3) == 2 ? x4.z : x4.w;
          ac[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(xv, wc[b][i], ac[a][b], 0, 0, 0);
        }
  };

  // the chains' block sums join the total in chain order and the block
  // starts again from zero
  auto fold = [&]() {
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int b = 0; b < WN; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            tot[a][b][r] += acc[c][a][b][r];
            acc[c][a][b][r] = 0.0f;
          }
        }
  };

  if (g0 < g1) {
#pragma unroll
    for (int u = 0; u < P; ++u) load(slot[u], std::min(g0 + u, g1 - 1));
  }
  // Whole rings: no branch between the loads, so the wait before each
  // consume counts only the loads issued after its slot's.  A block of
  // kAccGroups groups ends after a whole ring (P divides kAccGroups).
  static_assert(kAccGroups % P == 0, "blocks end on ring boundaries");
  int g = g0;
  for (; g + P <= g1; g += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      consume(slot[u], acc[u % CH]);
      load(slot[u], std::min(g + u + P, g1 - 1));
      // the reload stays here, right after the slot's last use: sunk below
      // the next slot's MFMAs it would shorten this slot's lead
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((g + P - g0) % kAccGroups == 0) fold();
  }
  // the last, partial ring
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (g + u < g1) consume(slot[u], acc[u % CH]);
  fold();

  if constexpr (KS > 1) {
    // Partial tiles of waves wk >= 1 go through LDS; wave wk == 0 adds them in
    // the order wk = 1, 2, ... and stores.
    extern __shared__ float red[];  // [KS-1][WAVES_MN][WM][WN][16][64]
    if (wk > 0) {
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[((((wk - 1) * WAVES_MN + wmn) * WM + a) * WN + b) * 1024 + r * 64 + lane] =
                tot[a][b][r];
    }
    __syncthreads();
    if (wk != 0) return;
    for (int k = 1; k < KS; ++k)
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tot[a][b][r] += red[((((k - 1) * WAVES_MN + wmn) * WM + a) * WN + b) * 1024 + r * 64 + lane];
  }

#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const int n = n_base + 32 * b + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m_base + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) Y[long(m) * N + n] = tot[a][b][r];
      }
    }
}

template <int WM, int WN, int BWM, int BWN, int KS, int P, int CH>
hipError_t run(const float *X, const int32_t *qw, const float *sc, float *Y, int M, int N, int G,
               hipStream_t stream) {
  constexpr int BM = 32 * WM * BWM, BN = 32 * WN * BWN;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const long blocks = long(tiles_m) * tiles_n;
  const size_t lds = KS > 1 ? size_t(KS - 1) * BWM * BWN * WM * WN * 1024 * sizeof(float) : 0;
  hipLaunchKernelGGL((tile_w4a16<WM, WN, BWM, BWN, KS, P, CH>), dim3(unsigned(blocks)),
                     dim3(64 * BWM * BWN * KS), lds, stream, X,
                     reinterpret_cast<const uint32_t *>(qw), sc, Y, M, N, G, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile(const float *X, const int32_t *qweight, const float *scales, float *Y,
                       int M, int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  // Large M: 128 x 128 block tiles, 4 waves of 64 x 64.
  const long big_tiles = long((M + 127) / 128) * ((N + 127) / 128);
  if (M > 64 && big_tiles >= 512)
    return run<2, 2, 2, 2, 1, kWidePrefetch, 1>(X, qweight, scales, Y, M, N, G, stream);
  // Otherwise 32 x 32 block tiles with the groups split over 8 waves: the
  // smallest tile gives the most blocks, so skinny shapes still fill all
  // compute units (M=64, N=4096: 256 blocks).
  return run<1, 1, 1, 1, kSkinnySplit, kSkinnyPrefetch, kSkinnyChains>(X, qweight, scales, Y, M,
                                                                       N, G, stream);
}

}  // namespace w4a16
