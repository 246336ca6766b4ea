// Split-precision path of the W4A16 GEMM: Y = X . dequant(W)^T on the fp16
// matrix cores, with fp32 accumulation and every product exact.
//
// The contraction the pages ask for is fp32 activations times int4 weights,
// accumulated in fp32 ("The Silence of Success: A Single Line That Speaks
// Volumes", sections "What the Edit Actually Built" and "Assumptions Embedded
// in the Code").  On gfx950 the fp32 matrix rate is 1/16 of the fp16 rate, so
// this path keeps the products exact and the accumulation fp32 while running
// on v_mfma_f32_16x16x32_f16:
//  * every weight code q - 8 (an integer in [-8, 7]) is exact in fp16;
//  * each activation row is scaled by a power of two 2^e so that its largest
//    magnitude lies in [2^14, 2^15), then split into two fp16 limbs
//    hi = f16(x'), lo = f16(x' - hi).  hi + lo equals x' to 22 significant
//    bits (relative error <= 2^-23; for elements below 2^-17 of the row's
//    largest, an absolute error <= 2^-25 * 2^-e);
//  * a product of two fp16 values is exact in fp32, and the MFMA accumulates
//    in fp32.  For one group of 32 k, the hi and the lo limbs are stacked along
//    the MFMA's K (two instructions into one accumulator, started from zero),
//    then the group's fp32 scale multiplies that group sum in one FMA into the
//    running fp32 sum; the row's 2^-e is applied exactly at the store.
//
// Kernels:
//  * split_prep: one workgroup per row of X: row maximum, exponent, limb
//    split; limbs are written in the order the weight conversion produces
//    (within each 8-wide k block: x0 x4 x1 x5 x2 x6 x3 x7).
//  * split_gemm<J>: block tile 64 (m) x 64 J (n), four waves of 64 x 16 J
//    (4 x J MFMA tiles of 16 x 16).  Work moves in stages of 2 groups whose
//    activation limbs, packed weights and scales are copied straight from
//    global memory into LDS, three stages deep.  Nibbles become f16 (q - 8)
//    pairs with a mask-or into the mantissa of 1024 (v_bitop3) and one packed
//    subtract (or a packed FMA for the nibbles that sit 4 bits up).  The MFMAs
//    of one (group, m-subtile) unit run while the previous unit's results are
//    scaled into the accumulators and the next unit's operands are read.
//  * The K range may be split over gridDim.y workgroups; each writes its
//    partial tile to the workspace and split_reduce adds the partials in split
//    order (deterministic), undoes the row's power of two and stores Y.

#include "w4a16_internal.h"
#include "limbs.h"

#include <algorithm>
#include <cmath>

namespace w4a16 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 64;      // rows of X / Y per workgroup tile

// ---------------------------------------------------------------- prep

constexpr int kPrepThreads = 256;
constexpr int kPrepRegBlocks = 4;  // 8-wide k blocks a thread keeps in registers

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// kInRegs: K <= 8 * 256 * kPrepRegBlocks, the row is read once and kept in
// registers; otherwise it is read twice (maximum, then split).
template <bool kInRegs>
__global__ void __launch_bounds__(kPrepThreads)
split_prep(const float *__restrict__ X, _Float16 *__restrict__ xl, int *__restrict__ rexp, int M,
           int K) {
  __shared__ float red[kPrepThreads / 64];
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const int K8 = K / 8;
  const float4 *xr = reinterpret_cast<const float4 *>(X + long(m) * K);
  half8_t *hi = reinterpret_cast<half8_t *>(xl + long(m) * K);
  half8_t *lo = reinterpret_cast<half8_t *>(xl + (long(M) + m) * K);
  float mx = 0.0f;
  if constexpr (kInRegs) {
    float4 a[kPrepRegBlocks], c[kPrepRegBlocks];
#pragma unroll
    for (int v = 0; v < kPrepRegBlocks; ++v) {
      const int b = t + v * kPrepThreads;
      a[v] = c[v] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (b < K8) {
        a[v] = xr[2 * b];
        c[v] = xr[2 * b + 1];
      }
    }
#pragma unroll
    for (int v = 0; v < kPrepRegBlocks; ++v)
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(fabsf(a[v].x), fabsf(a[v].y)),
                                 fmaxf(fabsf(a[v].z), fabsf(a[v].w))),
                           fmaxf(fmaxf(fabsf(c[v].x), fabsf(c[v].y)),
                                 fmaxf(fabsf(c[v].z), fabsf(c[v].w)))));
    const int e = row_exponent(block_max(mx, red));
    if (t == 0) rexp[m] = e;
#pragma unroll
    for (int v = 0; v < kPrepRegBlocks; ++v) {
      const int b = t + v * kPrepThreads;
      if (b < K8) {
        half8_t h, l;
        split_block(a[v], c[v], e, h, l);
        hi[b] = h;
        lo[b] = l;
      }
    }
  } else {
    for (int b = t; b < K8; b += kPrepThreads) {
      const float4 a = xr[2 * b], c = xr[2 * b + 1];
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w)))));
    }
    const int e = row_exponent(block_max(mx, red));
    if (t == 0) rexp[m] = e;
    for (int b = t; b < K8; b += kPrepThreads) {
      half8_t h, l;
      split_block(xr[2 * b], xr[2 * b + 1], e, h, l);
      hi[b] = h;
      lo[b] = l;
    }
  }
}

// ---------------------------------------------------------------- GEMM


// Work moves in stages of 2 groups (64 k).  A stage's operands are copied
// straight from global memory into LDS (global_load_lds), D stages deep, so
// that the copies of the next D - 1 stages are in flight while one stage is
// computed; no operand passes through registers on its way to LDS.  Per stage
// and workgroup (WN waves side by side along n, tile 64 x BN, BN = 16 J WN):
//  * A image, 16 KB: 2 limbs x 64 rows x 8 chunks of 16 bytes (8 f16 of k).
//    Chunk c of row r sits at slot c ^ ((r >> 1) & 7), so that the 16 rows an
//    MFMA operand read touches fall in 16 different bank groups.  Slot
//    u * T + t (T threads) is copied by thread t, copy u.
//  * W image, BN / 64 slabs of [group][row (64)][4 words]: lane (l16, kb)
//    reads word kb of its row with ds_read_b32, which is the B operand layout
//    (no cross-lane transpose).
//  * S image: [row][group] scales (at least one word per thread, so that every
//    thread issues the same number of copies and one wait count fits every
//    wave).
// The weights come either in the caller's layout (qweight, scales: each copy
// gathers 16 bytes of one row) or in the packed layout w4a16_split_pack
// writes, where a stage's weights and scales of a 64-row slab are contiguous
// (every copy reads whole cache lines).
constexpr int kStageK = 64;
constexpr int kSlab = 64;                // rows of W per slab
constexpr int kAImg = 2 * kBM * 8 * 16;  // bytes
constexpr int kPackW = 2 * kSlab * 16;   // packed bytes of weights per slab and stage
constexpr int kPackS = kSlab * 2 * 4;    // packed bytes of scales per slab and stage

template <int J, int WN>
struct StageLayout {
  static constexpr int kThreads = 64 * WN;
  static constexpr int kBN = WN * 16 * J;
  static constexpr int kSlabs = kBN / kSlab;
  static constexpr int kW = kSlabs * kPackW;  // bytes
  static constexpr int kSWords = 2 * kBN > kThreads ? 2 * kBN : kThreads;
  static constexpr int kS = kSWords * 4;  // bytes
  static constexpr int kBytes = kAImg + kW + kS;
  // copies per thread and stage: A 16 B each; W 16 B each, or 4 B each when the
  // W image is smaller than one 16-byte copy per thread; S 4 B each
  static constexpr int kACopies = kAImg / (kThreads * 16);
  static constexpr bool kWDword = kW < kThreads * 16;
  static constexpr int kWCopies = kWDword ? kW / (kThreads * 4) : kW / (kThreads * 16);
  static constexpr int kSCopies = kSWords / kThreads;
  static constexpr int kCopies = kACopies + kWCopies + kSCopies;
  static_assert(kBN % kSlab == 0 && kACopies >= 1, "tile shape");
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` stages of copies (issued after the one about to
// be read) are still in flight.
template <int kCopies, int kMaxAhead>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (kMaxAhead >= 2) {
    if (ahead >= 2) {
      wait_vmcnt<2 * kCopies>();
      return;
    }
  }
  if (ahead >= 1) {
    wait_vmcnt<kCopies>();
    return;
  }
  wait_vmcnt<0>();
}

// Workgroup barrier between stages.  __syncthreads() implies a release fence,
// which waits for every outstanding copy into LDS (vmcnt(0)) and so would
// drain the copies of the stages still ahead; here each wave has already
// waited for its own copies of the stage it is about to read, the LDS reads of
// the buffer the next copies overwrite were consumed in the previous stage, and
// the empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-thread sources of the copies that fill one stage's LDS image.
template <int J, int WN, bool kPacked>
struct StageCopier {
  using L = StageLayout<J, WN>;
  static constexpr int T = L::kThreads;
  const _Float16 *asrc[L::kACopies];
  const uint32_t *wsrc[L::kWCopies];
  int wgrp[L::kWCopies];
  const float *ssrc[L::kSCopies];
  long K;
  int c_col, G, stages, wave, t;

  __device__ __forceinline__ StageCopier(const _Float16 *xl, const uint32_t *qw, const float *sc,
                                         int M, int N, int G_, int m_base, int n_blk, int wave_,
                                         int t_)
      : K(long(G_) * kGroup), G(G_), stages((G_ + 1) / 2), wave(wave_), t(t_) {
    // A: copy u fills slot P = u * T + t: limb P / 512, row P / 8 % 64, chunk
    // column c (the same for every u: row / 2 % 8 = t / 16 % 8)
    c_col = (t & 7) ^ ((t >> 4) & 7);
#pragma unroll
    for (int u = 0; u < L::kACopies; ++u) {
      const int P = u * T + t;
      const int m = std::min(m_base + ((P >> 3) & (kBM - 1)), M - 1);
      asrc[u] = xl + (long(P >> 9) * M + m) * K;
    }
    // W: copy v covers image unit idx = v * T + t (16-byte chunk, or word):
    // chunk (slab, group, row) = (unit / 128, unit / 64 % 2, unit % 64)
    const int slab0 = n_blk / kSlab;
#pragma unroll
    for (int v = 0; v < L::kWCopies; ++v) {
      const int idx = v * T + t;
      const int unit = L::kWDword ? idx >> 2 : idx;
      const int word = L::kWDword ? (idx & 3) : 0;
      if constexpr (kPacked) {
        wsrc[v] = qw + ((long(slab0 + (unit >> 7)) * stages) * 128 + (unit & 127)) * 4 + word;
        wgrp[v] = 0;
      } else {
        const int n = std::min(n_blk + (unit >> 7) * kSlab + (unit & 63), N - 1);
        wsrc[v] = qw + long(n) * G * 4 + word;
        wgrp[v] = (unit >> 6) & 1;
      }
    }
    // S: copy v covers word idx = v * T + t of [row][group] (words past
    // 2 BN repeat the image and land in padding nobody reads)
#pragma unroll
    for (int v = 0; v < L::kSCopies; ++v) {
      const int idx = (v * T + t) & (2 * L::kBN - 1);
      if constexpr (kPacked) {
        ssrc[v] = sc + (long(slab0 + (idx >> 7)) * stages) * 128 + (idx & 127);
      } else {
        ssrc[v] = sc + long(std::min(n_blk + (idx >> 1), N - 1)) * G + (idx & 1);
      }
    }
  }

  // copies of stage st into the image at `base` (L::kCopies per thread)
  __device__ __forceinline__ void issue(unsigned char *__restrict__ base, int st) const {
    // a chunk past K reads the row's last chunk; its group's scale is 0
    const long k = std::min(long(st) * kStageK + c_col * 8, K - 8);
#pragma unroll
    for (int u = 0; u < L::kACopies; ++u)
      __builtin_amdgcn_global_load_lds(asrc[u] + k,
                                       (lds_void *)(base + (u * T + wave * 64) * 16), 16, 0, 0);
    unsigned char *wb = base + kAImg;
#pragma unroll
    for (int v = 0; v < L::kWCopies; ++v) {
      const uint32_t *src = kPacked ? wsrc[v] + long(st) * (128 * 4)
                                    : wsrc[v] + std::min(2 * st + wgrp[v], G - 1) * 4;
      if constexpr (L::kWDword)
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(wb + (v * T + wave * 64) * 4), 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(wb + (v * T + wave * 64) * 16), 16, 0,
                                         0);
    }
    unsigned char *sb = wb + L::kW;
#pragma unroll
    for (int v = 0; v < L::kSCopies; ++v) {
      const float *src;
      if constexpr (kPacked) {
        src = ssrc[v] + long(st) * 128;
      } else {
        // group 2 st + 1 past G (odd G): read group G - 1 instead, masked at use
        const int h = (v * T + t) & 1;
        src = ssrc[v] + std::min(2 * st + h, G - 1) - h;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(sb + (v * T + wave * 64) * 4), 4, 0, 0);
    }
  }
};

// One stage: 8 units (group g of the stage, m-subtile i); unit u's MFMAs run
// while unit u - 1's results are scaled into acc and unit u + 1's A operands
// are read.  `cur` is the image of this stage, `nxt` the buffer the copies of
// a later stage go to: distinct buffers, and the restrict qualifiers tell the
// compiler so (its own wait insertion then leaves these LDS reads alone; the
// explicit waits before the stage barrier order them).
template <int J, int WN, bool kPacked>
__device__ __forceinline__ void stage_compute(const unsigned char *__restrict__ cur,
                                              unsigned char *__restrict__ nxt, int st_next,
                                              const StageCopier<J, WN, kPacked> &cp, int st, int G,
                                              int wave, int l16, int kb, floatx4 (&acc)[4][J],
                                              floatx4 (&dp)[J], float (&sp)[J]) {
  using L = StageLayout<J, WN>;
  // this stage's weight words and scales into registers
  const unsigned char *wb = cur + kAImg;
  const unsigned char *sb = wb + L::kW;
  uint32_t w[J][2];
  float s[J][2];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int nl = wave * 16 * J + 16 * j + l16;
#pragma unroll
    for (int g = 0; g < 2; ++g)
      w[j][g] = *reinterpret_cast<const uint32_t *>(
          wb + (((nl / kSlab) * 2 + g) * kSlab + nl % kSlab) * 16 + kb * 4);
    const float2 sv = *reinterpret_cast<const float2 *>(sb + nl * 8);
    s[j][0] = sv.x;
    s[j][1] = 2 * st + 1 < G ? sv.y : 0.0f;  // odd G: the last stage has one group
  }
  if (st_next >= 0) cp.issue(nxt, st_next);

  auto a_addr = [&](int g, int i, int limb) {
    const int row = 16 * i + l16;
    const int slot = (g * 4 + kb) ^ ((row >> 1) & 7);
    return cur + ((limb * kBM + row) * 8 + slot) * 16;
  };
  half8_t ahi[2], alo[2];
  ahi[0] = *reinterpret_cast<const half8_t *>(a_addr(0, 0, 0));
  alo[0] = *reinterpret_cast<const half8_t *>(a_addr(0, 0, 1));
  half8_t b[J];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int g = u >> 2, i = u & 3, c = u & 1;
    if (i == 0) {
#pragma unroll
      for (int j = 0; j < J; ++j) b[j] = nibbles_to_f16(w[j][g]);
    }
    // The compiler waits for every outstanding LDS read (lgkmcnt(0)) before
    // the first use of any of them while copies into LDS are in flight, so
    // this unit first consumes both of its A operands (read during the
    // previous unit), and only then are the next unit's operands read.
    floatx4 d[J];
    d[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[c], b[0], floatx4{0.0f, 0.0f, 0.0f, 0.0f},
                                                  0, 0, 0);
    if constexpr (J > 1)
      d[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[c], b[1],
                                                    floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    else
      d[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[c], b[0], d[0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (u < 7) {  // next unit's A operands, read while this unit computes
      ahi[c ^ 1] = *reinterpret_cast<const half8_t *>(a_addr((u + 1) >> 2, (u + 1) & 3, 0));
      alo[c ^ 1] = *reinterpret_cast<const half8_t *>(a_addr((u + 1) >> 2, (u + 1) & 3, 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (J > 1) {
      d[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[c], b[0], d[0], 0, 0, 0);
      d[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[c], b[1], d[1], 0, 0, 0);
    }
#pragma unroll
    for (int j = 2; j < J; ++j) {
      d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[c], b[j], floatx4{0.0f, 0.0f, 0.0f, 0.0f},
                                                    0, 0, 0);
      d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[c], b[j], d[j], 0, 0, 0);
    }
    // the previous unit (m-subtile (i + 3) % 4; the one before a stage's
    // first unit is the last unit of the stage before) into acc
    const int pi = (i + 3) & 3;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[pi][j][r] = fmaf(dp[j][r], sp[j], acc[pi][j][r]);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      dp[j] = d[j];
      sp[j] = s[j][g];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Grid: x = output tile, y = K split.  Tiles are numbered m-tile major, n-tile
// minor; when their count divides by 8, workgroup b (the hardware deals
// workgroups round-robin to the 8 XCDs) takes tile (b % 8) * (tiles / 8) + b / 8,
// so that each XCD works through a contiguous run of tiles and its L2 serves
// the rows of X and W those tiles share.  D stage buffers: the copies of the
// next D - 1 stages are in flight while one is computed.  With kPacked, qw
// and sc point at the two regions of w4a16_split_pack's buffer.
template <int J, int WN, int D, bool kPacked>
__global__ void __launch_bounds__(64 * WN)
split_gemm(const _Float16 *__restrict__ xl, const int *__restrict__ rexp,
           const uint32_t *__restrict__ qw, const float *__restrict__ sc, float *__restrict__ Y,
           float *__restrict__ partial, int M, int N, int G, int n_tiles) {
  // device code only: the host pass needs no more than the launch signature
  // (it rejects instantiating the stage body for some template arguments)
#if defined(__HIP_DEVICE_COMPILE__)
  using L = StageLayout<J, WN>;
  constexpr int kBN = L::kBN;
  static_assert(D >= 2 && D <= 4 && (D - 2) * L::kCopies < 64, "pipeline depth");
  __shared__ __align__(16) unsigned char lds[D * L::kBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l16 = lane & 15;
  const int kb = lane >> 4;
  const int tiles = gridDim.x;
  int tile = blockIdx.x;
  if ((tiles & 7) == 0) tile = (tile & 7) * (tiles >> 3) + (tile >> 3);
  const int m_tile = tile / n_tiles;
  const int n_tile = tile - m_tile * n_tiles;
  const int split = blockIdx.y;
  const int S = gridDim.y;
  const int m_base = m_tile * kBM;
  const int n_blk = n_tile * kBN;
  const int stages = (G + 1) / 2;
  const int s0 = int((long(stages) * split) / S);
  const int s1 = int((long(stages) * (split + 1)) / S);
  const StageCopier<J, WN, kPacked> cp(xl, qw, sc, M, N, G, m_base, n_blk, wave, t);

  floatx4 acc[4][J];
  floatx4 dp[J];
  float sp[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    dp[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    sp[j] = 0.0f;
  }

#pragma unroll
  for (int k = 0; k < D - 1; ++k)
    if (s0 + k < s1) cp.issue(lds + ((s0 + k) % D) * L::kBytes, s0 + k);
  for (int st = s0; st < s1; ++st) {
    // stage st is in LDS (this wave's copies, then everyone's) and every wave
    // is done with the buffer that stage st + D - 1 goes to
    wait_stage<L::kCopies, D - 2>(std::min(st + D - 2, s1 - 1) - st);
    stage_barrier();
    const int nx = st + D - 1 < s1 ? st + D - 1 : -1;
    const unsigned char *cur = lds + (st % D) * L::kBytes;
    unsigned char *nxt = lds + ((st + D - 1) % D) * L::kBytes;
    stage_compute<J, WN, kPacked>(cur, nxt, nx, cp, st, G, wave, l16, kb, acc, dp, sp);
  }
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[3][j][r] = fmaf(dp[j][r], sp[j], acc[3][j][r]);

  // lane (l16, kb) of wave w holds rows m_base + 16 i + 4 kb + r of column
  // n_blk + 16 (J w + j) + l16.  One split: Y directly (the row's power of two
  // undone); several: this split's partial, still scaled, for split_reduce.
  float *out = S == 1 ? Y : partial + long(split) * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 16 * i + 4 * kb + r;
      if (m >= M) continue;
      const int e = S == 1 ? rexp[m] : 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int n = n_blk + wave * 16 * J + 16 * j + l16;
        if (n < N) out[long(m) * N + n] = ldexpf(acc[i][j][r], -e);
      }
    }
#endif
}

// Packed weights for the split path: for each slab of 64 rows and stage st,
// 128 chunks [group 2 st + g][row] of 4 words (2 KB), and in a second region
// 128 words of scales [row][group].  One thread per chunk; rows past N and the
// group past G (odd G) get code 0 (all nibbles 8) and scale 0.
__global__ void __launch_bounds__(256)
split_pack(const uint32_t *__restrict__ qw, const float *__restrict__ sc, uint4 *__restrict__ wp,
           float *__restrict__ sp, int N, int G, long chunks) {
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  if (i >= chunks) return;
  const int stages = (G + 1) / 2;
  const int c = int(i & 127);
  const long slab_stage = i >> 7;
  const int st = int(slab_stage % stages);
  const int slab = int(slab_stage / stages);
  const int g = c >> 6, r = c & 63;
  const int n = slab * kSlab + r, gg = 2 * st + g;
  const bool valid = n < N && gg < G;
  wp[i] = valid ? reinterpret_cast<const uint4 *>(qw)[long(n) * G + gg]
                : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
  sp[slab_stage * 128 + r * 2 + g] = valid ? sc[long(n) * G + gg] : 0.0f;
}

// Y = 2^-e(m) * (sum over splits in order of the partials): one float4 of
// outputs per thread when N % 4 == 0, else one output.  The partials' loads
// go out kBatch at a time before any of them is added (the adds stay in split
// order, so the result does not depend on the batching).
constexpr int kReduceBatch = 8;

template <bool kVec4>
__global__ void __launch_bounds__(256)
split_reduce(const float *__restrict__ partial, const int *__restrict__ rexp,
             float *__restrict__ Y, int M, int N, int S) {
  const long total = long(M) * N;
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  if constexpr (kVec4) {
    if (4 * i >= total) return;
    const float4 *p4 = reinterpret_cast<const float4 *>(partial);
    const long stride = total / 4;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int z0 = 0; z0 < S; z0 += kReduceBatch) {
      float4 p[kReduceBatch];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (z0 + u < S) p[u] = p4[long(z0 + u) * stride + i];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (z0 + u < S) {
          if (z0 + u == 0) {
            v = p[u];
          } else {
            v.x += p[u].x;
            v.y += p[u].y;
            v.z += p[u].z;
            v.w += p[u].w;
          }
        }
    }
    const int e = rexp[(4 * i) / N];
    reinterpret_cast<float4 *>(Y)[i] =
        make_float4(ldexpf(v.x, -e), ldexpf(v.y, -e), ldexpf(v.z, -e), ldexpf(v.w, -e));
  } else {
    if (i >= total) return;
    float v = 0.0f;
    for (int z0 = 0; z0 < S; z0 += kReduceBatch) {
      float p[kReduceBatch];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (z0 + u < S) p[u] = partial[long(z0 + u) * total + i];
#pragma unroll
      for (int u = 0; u < kReduceBatch; ++u)
        if (z0 + u < S) v = z0 + u == 0 ? p[u] : v + p[u];
    }
    Y[i] = ldexpf(v, -rexp[i / N]);
  }
}

struct SplitPlan {
  int J, WN, D, m_tiles, n_tiles, S;
  size_t off_exp, off_partial, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

SplitPlan make_plan(int M, int N, int G, int J, int WN, int S, int D) {
  SplitPlan p;
  p.J = J;
  p.WN = WN;
  p.D = D;
  p.S = S;
  p.m_tiles = (M + kBM - 1) / kBM;
  p.n_tiles = (N + WN * 16 * J - 1) / (WN * 16 * J);
  const size_t limbs = size_t(2) * M * size_t(G) * kGroup * sizeof(_Float16);
  p.off_exp = align256(limbs);
  p.off_partial = p.off_exp + align256(size_t(M) * sizeof(int));
  p.bytes = align256(p.off_partial + (S > 1 ? size_t(S) * M * size_t(N) * sizeof(float) : 0));
  return p;
}

// Tile shape and K split.  When 64 x 512 tiles already give every compute
// unit a workgroup, they are used unsplit (the widest tile moves the fewest
// activation bytes per MFMA).  Otherwise the K range is split (powers of two,
// at least 3 stages per split) until the grid covers the 256 compute units;
// among tile widths 256, 128 and 64 the one with the smallest estimated time
// wins, the estimate adding per-workgroup MFMA time, its L2 traffic and the
// split-K partials' round trip.
SplitPlan plan_split(int M, int N, int G) {
  const int stages = (G + 1) / 2;
  const int m_tiles = (M + kBM - 1) / kBM;
  if (long(m_tiles) * ((N + 511) / 512) >= 256) return make_plan(M, N, G, 4, 8, 1, 4);
  SplitPlan best{};
  double best_cost = 0.0;
  for (int J : {4, 2, 1}) {
    const int n_tiles = (N + 64 * J - 1) / (64 * J);
    int S = 1;
    while (long(m_tiles) * n_tiles * S < 256 && stages / (S * 2) >= 3) S *= 2;
    const double kq = double(stages) * kStageK / S;  // k per workgroup
    const double bn = 64.0 * J;
    const double mfma_us = kBM * bn * kq * 4.0 / 4.9e6;  // two limbs, ~half of peak
    // ~50 GB/s of L2-to-CU traffic per workgroup: what the K-split sweeps at
    // M = 64 measure once a workgroup's activation slice exceeds ~200 KB
    const double l2_us = (kBM * kq * 4.0 + bn * kq * 0.625) / 5e4;
    const double rounds = std::ceil(double(m_tiles) * n_tiles * S / 256.0);
    double cost = rounds * std::max(mfma_us, l2_us);
    if (S > 1) cost += 2.0 * S * double(M) * N * 4.0 / 5e6 + 1.2;
    if (J == 4 || cost < best_cost) {
      best = make_plan(M, N, G, J, 4, S, 3);
      best_cost = cost;
    }
  }
  return best;
}

template <bool kPacked>
hipError_t launch_gemm(const SplitPlan &p, const _Float16 *xl, const int *rexp, const void *wq,
                       const float *ws, float *Y, float *partial, int M, int N, int G,
                       hipStream_t stream) {
  const long tiles = long(p.m_tiles) * p.n_tiles;
  if (tiles > 0x7fffffffL || p.S > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(unsigned(tiles), unsigned(p.S));
  const auto qw = static_cast<const uint32_t *>(wq);
#define W4A16_SPLIT_GEMM(JJ, WW, DD)                                                             \
  hipLaunchKernelGGL((split_gemm<JJ, WW, DD, kPacked>), grid, dim3(64 * WW), 0, stream, xl, rexp,  \
                     qw, ws, Y, partial, M, N, G, p.n_tiles)
  switch (p.J * 100 + p.WN * 10 + p.D) {
    case 483: W4A16_SPLIT_GEMM(4, 8, 3); break;
    case 484: W4A16_SPLIT_GEMM(4, 8, 4); break;
    case 443: W4A16_SPLIT_GEMM(4, 4, 3); break;
    case 444: W4A16_SPLIT_GEMM(4, 4, 4); break;
    case 243: W4A16_SPLIT_GEMM(2, 4, 3); break;
    case 244: W4A16_SPLIT_GEMM(2, 4, 4); break;
    case 143: W4A16_SPLIT_GEMM(1, 4, 3); break;
    case 144: W4A16_SPLIT_GEMM(1, 4, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef W4A16_SPLIT_GEMM
  return hipGetLastError();
}

// prep, GEMM and (several splits) reduce; wq/ws: qweight and scales, or the
// two regions of a packed buffer
hipError_t launch_plan(const SplitPlan &p, bool packed, const float *X, const void *wq,
                       const float *ws, float *Y, int M, int N, int K, void *workspace,
                       hipStream_t stream) {
  const int G = K / kGroup;
  char *wsp = static_cast<char *>(workspace);
  _Float16 *xl = reinterpret_cast<_Float16 *>(wsp);
  int *rexp = reinterpret_cast<int *>(wsp + p.off_exp);
  float *partial = reinterpret_cast<float *>(wsp + p.off_partial);
  if (K <= 8 * kPrepThreads * kPrepRegBlocks)
    hipLaunchKernelGGL(split_prep<true>, dim3(M), dim3(kPrepThreads), 0, stream, X, xl, rexp, M,
                       K);
  else
    hipLaunchKernelGGL(split_prep<false>, dim3(M), dim3(kPrepThreads), 0, stream, X, xl, rexp, M,
                       K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = packed ? launch_gemm<true>(p, xl, rexp, wq, ws, Y, partial, M, N, G, stream)
             : launch_gemm<false>(p, xl, rexp, wq, ws, Y, partial, M, N, G, stream);
  if (e != hipSuccess || p.S == 1) return e;
  const long total = long(M) * N;
  if (N % 4 == 0) {
    const long blocks = (total / 4 + 255) / 256;
    hipLaunchKernelGGL(split_reduce<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, partial,
                       rexp, Y, M, N, p.S);
  } else {
    const long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(split_reduce<false>, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       partial, rexp, Y, M, N, p.S);
  }
  return hipGetLastError();
}

// the two regions of a packed buffer
void pack_regions(const void *packed, int N, int G, const uint32_t **wq, const float **ws) {
  const long slab_stages = long((N + kSlab - 1) / kSlab) * ((G + 1) / 2);
  *wq = static_cast<const uint32_t *>(packed);
  *ws = reinterpret_cast<const float *>(static_cast<const char *>(packed) + slab_stages * kPackW);
}

}  // namespace

size_t split_workspace_bytes(int M, int N, int K) { return plan_split(M, N, K / kGroup).bytes; }

hipError_t launch_split(const float *X, const int32_t *qweight, const float *scales, float *Y,
                        int M, int N, int K, void *workspace, hipStream_t stream) {
  return launch_plan(plan_split(M, N, K / kGroup), false, X, qweight, scales, Y, M, N, K,
                     workspace, stream);
}

size_t split_pack_bytes(int N, int K) {
  const long slab_stages = long((N + kSlab - 1) / kSlab) * ((K / kGroup + 1) / 2);
  return size_t(slab_stages) * (kPackW + kPackS);
}

hipError_t launch_split_pack(const int32_t *qweight, const float *scales, void *packed, int N,
                             int K, hipStream_t stream) {
  const int G = K / kGroup;
  const long chunks = long((N + kSlab - 1) / kSlab) * ((G + 1) / 2) * 128;
  const uint32_t *wq;
  const float *ws;
  pack_regions(packed, N, G, &wq, &ws);
  hipLaunchKernelGGL(split_pack, dim3(unsigned((chunks + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t *>(qweight), scales,
                     reinterpret_cast<uint4 *>(const_cast<uint32_t *>(wq)),
                     const_cast<float *>(ws), N, G, chunks);
  return hipGetLastError();
}

hipError_t launch_split_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                               void *workspace, hipStream_t stream) {
  const uint32_t *wq;
  const float *ws;
  pack_regions(packed, N, K / kGroup, &wq, &ws);
  return launch_plan(plan_split(M, N, K / kGroup), true, X, wq, ws, Y, M, N, K, workspace,
                     stream);
}

size_t split_workspace_bytes_with(int M, int N, int K, int J, int WN, int S) {
  return make_plan(M, N, K / kGroup, J, WN, S, 3).bytes;
}

hipError_t launch_split_with(const float *X, const void *weights, const float *scales, bool packed,
                             float *Y, int M, int N, int K, int J, int WN, int S, int D,
                             void *workspace, hipStream_t stream) {
  if (S < 1) return hipErrorInvalidValue;
  const SplitPlan p = make_plan(M, N, K / kGroup, J, WN, S, D);
  if (packed) {
    const uint32_t *wq;
    const float *ws;
    pack_regions(weights, N, K / kGroup, &wq, &ws);
    return launch_plan(p, true, X, wq, ws, Y, M, N, K, workspace, stream);
  }
  return launch_plan(p, false, X, weights, scales, Y, M, N, K, workspace, stream);
}

}  // namespace w4a16
