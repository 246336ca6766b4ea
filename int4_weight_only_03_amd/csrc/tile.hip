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
#ifndef W4A16_TILE_LDS
#define W4A16_TILE_LDS 1
#endif
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

// ---------------------------------------------------------------------------
// The 128 x 128 tile with its operands staged in LDS (large M).
//
// The same arithmetic and accumulation order as tile_w4a16<2, 2, 2, 2, 1>
// (exact dequantized fp32 weights, v_mfma_f32_32x32x2_f32, block sums of
// kAccGroups groups), with the loads reorganised: loading each lane's own
// operands took 32 rows per load instruction (one L1 access each), and the
// address stage waited on the L1 for 30% of the kernel.  Here the workgroup's
// 4 waves copy each group's 128 rows of X (128 B per row) into LDS together,
// 1 KB per copy instruction (global_load_lds), and the weight words and
// scales of 4 groups at a time (64 B and 16 B per row); each wave then reads
// its MFMA operands from LDS.  Two X images and two weight/scale images
// alternate; the copies of group g + 1 (and, every 4 groups, of the next 4
// groups' weights) are issued right after the barrier that opens group g, so
// they land under group g's MFMAs.
//
// k order: lane (l32, h) supplies k = 16h .. 16h + 15 of its group, A from
// LDS chunks 4h .. 4h+3 of its X row, B from words 2h, 2h+1 of its W row.
// X rows are XOR-swizzled (chunk ^ ((row >> 1) & 7)) and each W row's four
// groups too (group ^ ((row >> 2) & 3)), so the operand reads are free of bank
// conflicts; a lane's read addresses are then one base XOR the chunk or group.

typedef __attribute__((address_space(3))) void tl_lds_void;

__device__ __forceinline__ void tl_wait_vm0() {
  __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | 0x70 | (15 << 8));  // vmcnt(0)
}
__device__ __forceinline__ void tl_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | 0x70);  // lgkmcnt(0)
}
// Workgroup barrier.  __syncthreads() would add a release fence that waits for
// every copy in flight (vmcnt(0)), the next group's included; each wave has
// already waited for its own copies of the group about to be read.
__device__ __forceinline__ void tl_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(256)
tile_lds(const float *__restrict__ X, const uint32_t *__restrict__ qw,
         const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G, int tiles_n) {
  // distinct LDS objects: the compiler can tell a read of one image from the
  // copies into the other (else it waits for every copy before any read)
  __shared__ __align__(16) unsigned char tl_x0[128 * 128];
  __shared__ __align__(16) unsigned char tl_x1[128 * 128];
  __shared__ __align__(16) unsigned char tl_w0[128 * 64];
  __shared__ __align__(16) unsigned char tl_w1[128 * 64];
  __shared__ __align__(16) unsigned char tl_s0[128 * 16];
  __shared__ __align__(16) unsigned char tl_s1[128 * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
#ifndef W4A16_TILE_XCD
#define W4A16_TILE_XCD 1
#endif
  int tile = blockIdx.x;
  if (W4A16_TILE_XCD && gridDim.x % 8 == 0) {
    // the hardware deals workgroups round-robin to the 8 XCDs: XCD x takes
    // the contiguous run of tiles x * (tiles / 8) ..
    tile = int(blockIdx.x % 8) * int(gridDim.x / 8) + int(blockIdx.x / 8);
  }
  const int bm = tile / tiles_n;
  const int bn = tile - bm * tiles_n;
  const int m0 = bm * 128, n0 = bn * 128;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const long K = long(G) * kGroup;

  // X copy j (this wave issues j = 4 wave .. 4 wave + 3): lane i writes 16 B
  // at image offset 1024 j + 16 i: tile row 8j + i/8, physical chunk i % 8,
  // holding logical chunk (i % 8) ^ ((row >> 1) & 7) of the group's 128 B.
  // Offsets relative to the tile's first row (below 2^26); rows past M read
  // row M-1 (never stored).
  uint32_t xoff[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int row = 8 * (4 * wave + jj) + lane / 8;
    const int L = (lane & 7) ^ ((row >> 1) & 7);
    xoff[jj] = uint32_t(std::min(m0 + row, M - 1) - m0) * uint32_t(K * 4) + 16u * uint32_t(L);
  }
  const char *xtile = reinterpret_cast<const char *>(X) + long(m0) * K * 4;
  // W copy c (this wave issues c = 2 wave, 2 wave + 1): lane i writes 16 B at
  // offset 1024 c + 16 i: tile row 16c + i/4, position i % 4, which holds group
  // (i % 4) ^ ((row / 4) % 4) of the block.  Scale copy c: lane i writes 4 B at
  // offset 256 c + 4 i: the scale of group i % 4 of the same row.  Rows past N
  // read row N-1.
  uint32_t woff[2], soff[2];
  int wgr[2];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int row = 16 * (2 * wave + cc) + lane / 4;
    wgr[cc] = (lane & 3) ^ ((row >> 2) & 3);
    const uint32_t r = uint32_t(std::min(n0 + row, N - 1) - n0);
    woff[cc] = (r * uint32_t(G) + uint32_t(wgr[cc])) * 16u;
    soff[cc] = (r * uint32_t(G) + uint32_t(lane & 3)) * 4u;
  }
  const char *wtile = reinterpret_cast<const char *>(qw) + long(n0) * G * 16;
  const char *stile = reinterpret_cast<const char *>(sc) + long(n0) * G * 4;
  // this lane's operand read bases in the images: A rows wm*64 + 32a + l32
  // (chunk 4h, swizzled), W rows wn*64 + 32b + l32 (words 2h, 2h+1 of group 0,
  // swizzled) and their scales
  uint32_t xbo[2], wbo[2], sbo[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = wm * 64 + 32 * a + l32;
    xbo[a] = uint32_t(r * 128 + 16 * ((4 * h) ^ ((r >> 1) & 7)));
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int n = wn * 64 + 32 * b + l32;
    wbo[b] = uint32_t(n * 64 + 16 * ((n >> 2) & 3) + 8 * h);
    sbo[b] = uint32_t(n * 16);
  }

  auto load_x = [&](unsigned char *img, int g) {
    const char *base = xtile + long(g) * 128;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const char *src = base + xoff[jj];
      __builtin_amdgcn_global_load_lds(src, (tl_lds_void *)(img + 1024 * (4 * wave + jj)), 16, 0, 0);
    }
  };
  // the weights and scales of groups 4 blk .. 4 blk + 3 (groups past G re-read
  // group G-1; never used)
  auto load_ws = [&](unsigned char *wimg, unsigned char *simg, int blk) {
    const long gb = 4L * blk;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = 2 * wave + cc;
      const long gw = std::min(gb + wgr[cc], long(G) - 1);
      const char *wsrc = wtile + gw * 16 + (woff[cc] - 16u * uint32_t(wgr[cc]));
      __builtin_amdgcn_global_load_lds(wsrc, (tl_lds_void *)(wimg + 1024 * c), 16, 0, 0);
      const long gs = std::min(gb + (lane & 3), long(G) - 1);
      const char *ssrc = stile + gs * 4 + (soff[cc] - 4u * uint32_t(lane & 3));
      __builtin_amdgcn_global_load_lds(ssrc, (tl_lds_void *)(simg + 256 * c), 4, 0, 0);
    }
  };

  floatx16 acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = tot[a][b][r] = 0.0f;

  // the dequantized weights of one group: wc[b][i] = fl32((q - 8) * s) for W
  // row wn*64 + 32b + l32, k = 16h + i (group gq = g % 4 of images wimg, simg)
  auto dequant = [&](const unsigned char *wimg, const unsigned char *simg, int gq,
                     float (&wc)[2][16]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = wn * 64 + 32 * b + l32;
      const int pos = gq ^ ((n >> 2) & 3);
      const uint2 wv = *reinterpret_cast<const uint2 *>(wimg + n * 64 + pos * 16 + 8 * h);
      const float s = *reinterpret_cast<const float *>(simg + n * 16 + 4 * gq);
      const float neg8s = -8.0f * s;
      const uint32_t u[2] = {wv.x, wv.y};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // word 2h + t holds k = 16h + 8t .. 16h + 8t + 7, nibble i at bits 4i
        const uint32_t lo = u[t] & 0x0F0F0F0Fu;         // nibbles 0, 2, 4, 6
        const uint32_t hi = (u[t] >> 4) & 0x0F0F0F0Fu;  // nibbles 1, 3, 5, 7
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // (q - 8) * s rounded once: q*s - 8s is exact before the FMA's rounding
          wc[b][8 * t + 2 * bb] = fmaf(float((lo >> (8 * bb)) & 0xFFu), s, neg8s);
          wc[b][8 * t + 2 * bb + 1] = fmaf(float((hi >> (8 * bb)) & 0xFFu), s, neg8s);
        }
      }
    }
  };
  // this group's 64 MFMAs (A from image ximg, B = wc), and under them the next
  // group's dequantization into wn_ (when there is a next group): its weight
  // words and scales are read first, then each quarter of the MFMAs (one
  // float4 of A per row tile) is followed by a quarter of the dequantization
  // (one word of one W row), pinned there, so the conversions issue while
  // the matrix core works.
  auto step = [&](const unsigned char *ximg, const float (&wc)[2][16], bool more,
                  const unsigned char *wimg_n, const unsigned char *simg_n, int gq_n,
                  float (&wn_)[2][16]) {
    uint2 wv[2];
    float sv[2];
    if (more) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // byte offset of group 0's words 2h, 2h+1 of row n; group gq_n is at
        // that offset XOR 16 gq_n (the row's groups are XOR-swizzled)
        const uint32_t o = (wbo[b] ^ (16u * uint32_t(gq_n)));
        wv[b] = *reinterpret_cast<const uint2 *>(wimg_n + o);
        sv[b] = *reinterpret_cast<const float *>(simg_n + sbo[b] + 4 * gq_n);
      }
    }
    // A: chunk 4h + v of row r sits at (r*128 + 16*(4h ^ key)) XOR 16 v
    auto read_a = [&](int a, int v) {
      return *reinterpret_cast<const float4 *>(ximg + (xbo[a] ^ (16u * uint32_t(v))));
    };
    float4 xa[2][2];  // A of quarter v (both row tiles), double-buffered
    xa[0][0] = read_a(0, 0);
    xa[0][1] = read_a(1, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v < 3) {
        xa[(v + 1) & 1][0] = read_a(0, v + 1);
        xa[(v + 1) & 1][1] = read_a(1, v + 1);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * v + c;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const float4 &x4 = xa[v & 1][a];
          const float xv = c == 0 ? x4.x : c == 1 ? x4.y : c == 2 ? x4.z : x4.w;
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(xv, wc[b][i], acc[a][b], 0, 0, 0);
        }
      }
      if (more) {
        // quarter v of the next group's weights: word t = v % 2 of W row tile b = v / 2
        const int b = v >> 1, t = v & 1;
        const float s = sv[b];
        const float neg8s = -8.0f * s;
        const uint32_t w = t == 0 ? wv[b].x : wv[b].y;
        const uint32_t lo = w & 0x0F0F0F0Fu;         // nibbles 0, 2, 4, 6
        const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 1, 3, 5, 7
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // (q - 8) * s rounded once: q*s - 8s is exact before the FMA's rounding
          wn_[b][8 * t + 2 * bb] = fmaf(float((lo >> (8 * bb)) & 0xFFu), s, neg8s);
          wn_[b][8 * t + 2 * bb + 1] = fmaf(float((hi >> (8 * bb)) & 0xFFu), s, neg8s);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: group 0's X and the first block's weights and scales
  load_x(tl_x0, 0);
  load_ws(tl_w0, tl_s0, 0);
  float wq[2][2][16];  // dequantized weights of the current and the next group
  // every wave's copies of the first block must have landed: each wave
  // dequantizes rows that other waves copied
  asm volatile("" ::: "memory");
  tl_wait_vm0();
  tl_barrier();
  dequant(tl_w0, tl_s0, 0, wq[0]);
  // Blocks of kAccGroups = 8 groups: X images alternate per group, weight
  // images per 4 groups; the block sum joins the total after each block.
  static_assert(kAccGroups == 8, "the loop body is one block of 8 groups");
  for (int gb = 0; gb < G; gb += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = gb + u;
      if (g < G) {
        unsigned char *xcur = (u & 1) ? tl_x1 : tl_x0;
        unsigned char *xnext = (u & 1) ? tl_x0 : tl_x1;
        unsigned char *wnext = (u & 4) ? tl_w0 : tl_w1;
        unsigned char *snext = (u & 4) ? tl_s0 : tl_s1;
        // the next group's weight images: the same 4-group block, or the next
        unsigned char *wn1 = ((u + 1) & 4) ? tl_w1 : tl_w0;
        unsigned char *sn1 = ((u + 1) & 4) ? tl_s1 : tl_s0;
        // this wave's copies of group g are done; after the barrier, every
        // wave's are, and every wave is past group g - 1 (whose images the
        // copies below overwrite)
        asm volatile("" ::: "memory");
        tl_wait_vm0();
        tl_wait_lgkm0();
        tl_barrier();
        if (g + 1 < G) load_x(xnext, g + 1);
        if ((u & 3) == 0 && g + 4 < G) load_ws(wnext, snext, g / 4 + 1);
        __builtin_amdgcn_sched_barrier(0);
        step(xcur, wq[u & 1], g + 1 < G, wn1, sn1, (u + 1) & 3, wq[(u + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tot[a][b][r] += acc[a][b][r];
          acc[a][b][r] = 0.0f;
        }
  }

  const int mb = m0 + wm * 64, nb = n0 + wn * 64;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = nb + 32 * b + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
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
  if (M > 64 && big_tiles >= 512) {
#if W4A16_TILE_LDS
    if (big_tiles > 0x7fffffffL) return hipErrorInvalidValue;
    const int tiles_n = (N + 127) / 128;
    hipLaunchKernelGGL(tile_lds, dim3(unsigned(big_tiles)), dim3(256), 0, stream, X,
                       reinterpret_cast<const uint32_t *>(qweight), scales, Y, M, N, G, tiles_n);
    return hipGetLastError();
#else
    return run<2, 2, 2, 2, 1, kWidePrefetch, 1>(X, qweight, scales, Y, M, N, G, stream);
#endif
  }
  // Otherwise 32 x 32 block tiles with the groups split over 8 waves: the
  // smallest tile gives the most blocks, so skinny shapes still fill all
  // compute units (M=64, N=4096: 256 blocks).
  return run<1, 1, 1, 1, kSkinnySplit, kSkinnyPrefetch, kSkinnyChains>(X, qweight, scales, Y, M,
                                                                       N, G, stream);
}

}  // namespace w4a16
