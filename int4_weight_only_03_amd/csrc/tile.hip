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
// For one group of 32 k, lane (l%32, h = l/32) owns the 16 consecutive k
// 32g+16h .. 32g+16h+15: 16 activations (four 16-byte loads of one X row)
// and 16 nibbles (one 8-byte load, words 4g+2h and 4g+2h+1 of one W row), and
// the 16 MFMAs of the group each consume one of them.  Dequantization goes
// straight into the B registers: no LDS round trip, since the wave that
// dequantizes a weight is the wave that consumes it.
//
// A wave computes (32*WM) x (32*WN) outputs; a block has BWM x BWN such waves
// side by side and KS copies of that arrangement splitting the groups; the KS
// partial tiles are summed in LDS in a fixed order (deterministic, no atomics).
// The next group's raw loads are issued before the current group's MFMAs.
//
// Accumulation order.  The MFMAs of kAccGroups consecutive groups (16 each)
// accumulate from zero into a block sum, and each block sum is added to the
// running total with one fp32 add.  A single chain over all of K would let
// the rounding error of sign-coherent products (every x*w >= 0) grow with the
// chain length until it leaves the tolerance near K = 2^17; with blocks of
// 8 groups the longest chain is 128 MFMAs plus K/256 block adds.

#include "w4a16_internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kAccGroups = 8;  // groups per block sum (see "Accumulation order")

template <int WM, int WN, int BWM, int BWN, int KS>
__global__ void __launch_bounds__(64 * BWM * BWN * KS)
tile_w4a16(const float *__restrict__ X, const uint32_t *__restrict__ qw,
           const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G,
           int tiles_n) {
  constexpr int BM = 32 * WM * BWM;
  constexpr int BN = 32 * WN * BWN;
  constexpr int WAVES_MN = BWM * BWN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
    xrow[a] = X + long(m) * K + 16 * h;
  }
  const uint2 *qrow[WN];
  const float *srow[WN];
#pragma unroll
  for (int b = 0; b < WN; ++b) {
    const int n = std::min(n_base + 32 * b + l32, N - 1);
    qrow[b] = reinterpret_cast<const uint2 *>(qw + long(n) * (long(G) * 4)) + h;
    srow[b] = sc + long(n) * G;
  }

  floatx16 acc[WM][WN];  // block sum of the current kAccGroups groups
  floatx16 tot[WM][WN];  // sum of the finished blocks
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = tot[a][b][r] = 0.0f;

  float4 xa[WM][4];
  uint2 wq[WN];
  float ws[WN];
  auto load = [&](int g) {
#pragma unroll
    for (int a = 0; a < WM; ++a) {
      const float4 *p = reinterpret_cast<const float4 *>(xrow[a] + long(g) * kGroup);
#pragma unroll
      for (int v = 0; v < 4; ++v) xa[a][v] = p[v];
    }
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      wq[b] = qrow[b][2 * g];
      ws[b] = srow[b][g];
    }
  };

  if (g0 < g1) load(g0);
  for (int g = g0; g < g1; ++g) {
    float xc[WM][16];
    float wc[WN][16];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        xc[a][4 * v + 0] = xa[a][v].x;
        xc[a][4 * v + 1] = xa[a][v].y;
        xc[a][4 * v + 2] = xa[a][v].z;
        xc[a][4 * v + 3] = xa[a][v].w;
      }
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const float s = ws[b];
      const float neg8s = -8.0f * s;
      const uint32_t u[2] = {wq[b].x, wq[b].y};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t lo = u[w] & 0x0F0F0F0Fu;         // nibbles 0,2,4,6 of the word
        const uint32_t hi = (u[w] >> 4) & 0x0F0F0F0Fu;  // nibbles 1,3,5,7
#pragma unroll
        for (int byte = 0; byte < 4; ++byte) {
          const float q0 = float((lo >> (8 * byte)) & 0xFFu);
          const float q1 = float((hi >> (8 * byte)) & 0xFFu);
          // (q - 8) * s rounded once: q*s - 8s is exact before the FMA's rounding
          wc[b][8 * w + 2 * byte + 0] = fmaf(q0, s, neg8s);
          wc[b][8 * w + 2 * byte + 1] = fmaf(q1, s, neg8s);
        }
      }
    }
    if (g + 1 < g1) load(g + 1);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(xc[a][i], wc[b][i], acc[a][b], 0, 0, 0);
    // at the end of each block of kAccGroups groups (and of the range) the
    // block sum joins the total and the next block starts from zero
    if ((g - g0) % kAccGroups == kAccGroups - 1 || g + 1 == g1) {
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            tot[a][b][r] += acc[a][b][r];
            acc[a][b][r] = 0.0f;
          }
    }
  }

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

template <int WM, int WN, int BWM, int BWN, int KS>
hipError_t run(const float *X, const int32_t *qw, const float *sc, float *Y, int M, int N, int G,
               hipStream_t stream) {
  constexpr int BM = 32 * WM * BWM, BN = 32 * WN * BWN;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const long blocks = long(tiles_m) * tiles_n;
  const size_t lds = KS > 1 ? size_t(KS - 1) * BWM * BWN * WM * WN * 1024 * sizeof(float) : 0;
  hipLaunchKernelGGL((tile_w4a16<WM, WN, BWM, BWN, KS>), dim3(unsigned(blocks)),
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
    return run<2, 2, 2, 2, 1>(X, qweight, scales, Y, M, N, G, stream);
  // Otherwise 32 x 32 block tiles with the groups split over 8 waves: the
  // smallest tile gives the most blocks, so skinny shapes still fill all
  // compute units (M=64, N=4096: 256 blocks).
  return run<1, 1, 1, 1, 8>(X, qweight, scales, Y, M, N, G, stream);
}

}  // namespace w4a16
