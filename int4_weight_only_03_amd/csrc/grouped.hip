// Grouped (mixture-of-experts) W4A16 GEMM: many experts in one launch, each
// with its own, possibly empty, set of rows of X.
//
// The pages run the MoE experts, the shared expert and the dense MLP through
// the INT4 path ("The Quiet Commit: How a Single Documentation Edit Marks the
// Completion of a Major Engineering Milestone", section "The INT4
// Milestone"), name a Marlin MoE kernel as the production plan, and build the
// path for memory-bound MoE inference ("The Quiet Commit: How a Single Plan
// Update Closed Phase 3 of a Native DDTree Inference Engine", section "Input
// and Output Knowledge").  In decode each expert sees a handful of tokens, so
// the work per expert is a small-M GEMV over that expert's weights, and the
// whole launch is bound by reading every active expert's weights once.
//
// Inputs: tokens X[T][K]; R routed slots sorted by expert, slot r reading
// token token_index[r]; expert_offsets[E+1], expert e owning slots
// [expert_offsets[e], expert_offsets[e+1]); expert weights qweight[E][N][K/8]
// and scales[E][N][K/32].  Output Y[R][N]: Y[r] = X[token_index[r]] .
// dequant(W_e)^T for the expert e owning slot r.
//
// Grid: x = row blocks of an expert, y = expert.  A block reads its
// expert's slot range first and leaves at once when the expert has no slot,
// so empty experts cost one tiny block each and their weights are never
// read.  Otherwise (main kernel, grouped_rows) the block stages the token
// rows of up to MT slots in LDS once, and each wave streams whole weight
// rows: lane l takes groups l, l+64, ... of RB rows at a time, all of their
// 16-byte loads issued before any is used, applies each group's staged
// activations to all RB rows (signed-byte dequant, group sum times scale, as
// in the GEMV kernels), and a DPP sum over the wave gives each output.  When
// MT token rows do not fit in LDS, gemv_grouped reads activations straight
// from memory with LDS team reductions instead.  Slot offsets and token
// indices come from device memory; they are clamped into range before any
// use, so malformed routing gives wrong values, never an out-of-bounds
// access.  Every output is summed in a fixed order (deterministic).

#include "w4a16_internal.h"
#include "gemv_common.h"
#include "limbs.h"

#include <algorithm>
#include <atomic>

namespace w4a16 {
namespace {

constexpr int kMaxBlockG = 512;

template <int MT, int RB>
__global__ void __launch_bounds__(kMaxBlockG)
gemv_grouped(const float *__restrict__ X, const int32_t *__restrict__ token_index,
             const int32_t *__restrict__ offsets, const uint4 *__restrict__ qw,
             const float *__restrict__ sc, float *__restrict__ Y, int T, int R, int N, int G,
             int S, int TPS, int TR) {
  extern __shared__ float red[];  // [MT*RB][blockDim.x + 1]
  const int e = blockIdx.y;
  const int r0 = std::min(std::max(offsets[e], 0), R);
  const int r1 = std::min(std::max(offsets[e + 1], r0), R);
  const int me = r1 - r0;  // slots of this expert
  if (me == 0) return;     // uniform over the block
  const int BS = blockDim.x;
  const int ld = BS + 1;
  const int t = threadIdx.x;
  const int slot = t / TPS;
  const int col = t - slot * TPS;
  const bool active = slot < S;
  const long rowbase = long(blockIdx.x) * S * RB;
  const long K = long(G) * kGroup;
  const uint4 *qwe = qw + long(e) * N * G;
  const float *sce = sc + long(e) * N * G;

  for (int m0 = 0; m0 < me; m0 += MT) {
    float acc[MT][RB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[m][i] = 0.0f;
    const float *xrow[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {  // slots past the expert's range are computed and dropped
      const int tok = token_index[r0 + std::min(m0 + m, me - 1)];
      xrow[m] = X + long(std::min(std::max(tok, 0), T - 1)) * K;
    }

    if (active) {
      for (int g = col; g < G; g += TPS) {
        uint4 w[RB];
        float s[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {  // clamped rows: no branch between loads
          const long n = std::min(rowbase + slot + long(i) * S, long(N) - 1);
          w[i] = load_stream16(qwe + n * G + g);
          s[i] = load_stream4(sce + n * G + g);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float x[32];
          const float4 *xp = reinterpret_cast<const float4 *>(xrow[m] + long(g) * kGroup);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const float4 f = xp[v];
            x[4 * v + 0] = f.x;
            x[4 * v + 1] = f.y;
            x[4 * v + 2] = f.z;
            x[4 * v + 3] = f.w;
          }
#pragma unroll
          for (int i = 0; i < RB; ++i)
            acc[m][i] = fmaf(s[i], group_dot16(x, w[i]) * 0.0625f, acc[m][i]);
        }
      }
    }

#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i) red[(m * RB + i) * ld + t] = acc[m][i];
    __syncthreads();

    const int O = MT * S * RB;  // outputs of this block and slot chunk
    const int team = t / TR;
    const int j = t - team * TR;
    const int teams = BS / TR;
    for (int o = team; o < O; o += teams) {
      const int m = o / (S * RB);
      const int r = o - m * S * RB;
      const int i = r / S;
      const int sl = r - i * S;
      const float *src = red + (m * RB + i) * ld + sl * TPS;
      float v = 0.0f;
      for (int c = j; c < TPS; c += TR) v += src[c];
      for (int d = TR >> 1; d > 0; d >>= 1) v += __shfl_xor(v, d, TR);
      const long n = rowbase + sl + long(i) * S;
      if (j == 0 && m0 + m < me && n < N) Y[long(r0 + m0 + m) * N + n] = v;
    }
    __syncthreads();
  }
}

constexpr int kRowsThreads = 256;       // 4 waves
constexpr int kRowsMaxLds = 64 * 1024;  // staged token rows, bytes
constexpr int kGL = 4;                   // groups per lane per pass (64 * kGL groups)
constexpr int kStage = 8;                // 16-byte staging loads per thread in flight

// Staged rows keep each group's eight float4 together but rotate their order
// by the group index (slot v of group g at v ^ (g % 8)): a lane reads one
// group, so the lanes of one read would otherwise all sit 128 bytes apart on
// the same LDS banks.
__device__ __forceinline__ int x_slot(int q) { return (q & ~7) | ((q ^ (q >> 3)) & 7); }

template <int MT, int RB>
__global__ void __launch_bounds__(kRowsThreads)
grouped_rows(const float *__restrict__ X, const int32_t *__restrict__ token_index,
             const int32_t *__restrict__ offsets, const uint4 *__restrict__ qw,
             const float *__restrict__ sc, float *__restrict__ Y, int T, int R, int N, int G,
             int rows_per_block) {
  extern __shared__ __align__(16) float xs[];  // [MT][K] staged token rows
  const int e = blockIdx.y;
  const int r0 = std::min(std::max(offsets[e], 0), R);
  const int r1 = std::min(std::max(offsets[e + 1], r0), R);
  const int me = r1 - r0;
  const int n_begin = blockIdx.x * rows_per_block;
  if (me == 0 || n_begin >= N) return;  // uniform over the block
  const int n_end = std::min(N, n_begin + rows_per_block);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const long K = long(G) * kGroup;
  const uint4 *qwe = qw + long(e) * N * G;
  const float *sce = sc + long(e) * N * G;
  const int K4 = G * 8;  // float4 per token row

  for (int m0 = 0; m0 < me; m0 += MT) {
    const float4 *xrow[MT];  // the chunk's token rows (slots past the range repeat the last)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int tok = token_index[r0 + std::min(m0 + m, me - 1)];
      xrow[m] = reinterpret_cast<const float4 *>(X + long(std::min(std::max(tok, 0), T - 1)) * K);
    }
    __syncthreads();  // the previous chunk's rows are no longer read
    // stage the rows: kStage independent 16-byte loads per thread in flight
    // (clamped indices, straight-line), then the stores
    float4 *xs4 = reinterpret_cast<float4 *>(xs);
#pragma unroll
    for (int m = 0; m < MT; ++m)
      for (int k0 = t; k0 < K4; k0 += kRowsThreads * kStage) {
        float4 v[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) v[u] = xrow[m][std::min(k0 + u * kRowsThreads, K4 - 1)];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
          const int q = k0 + u * kRowsThreads;  // float4 q of the row: group q/8, slot q%8
          if (q < K4) xs4[m * K4 + x_slot(q)] = v[u];
        }
      }
    __syncthreads();
    for (int n0 = n_begin + wave * RB; n0 < n_end; n0 += 4 * RB) {
      float acc[MT][RB];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[m][i] = 0.0f;
      for (int gb = 0; gb < G; gb += 64 * kGL) {
        uint4 w[kGL][RB];
        float s[kGL][RB];
#pragma unroll
        for (int j = 0; j < kGL; ++j)  // every load of the pass issued first
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const int g = std::min(gb + lane + 64 * j, G - 1);
            const long n = std::min(n0 + i, N - 1);
            w[j][i] = load_stream16(qwe + n * G + g);
            s[j][i] = load_stream4(sce + n * G + g);
          }
#pragma unroll
        for (int j = 0; j < kGL; ++j) {
          const int g = gb + lane + 64 * j;
          const bool valid = g < G;  // groups past G weigh nothing
          const int gc = valid ? g : G - 1;
          float x[MT][32];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float4 *xp = reinterpret_cast<const float4 *>(xs + m * K + long(gc) * kGroup);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              const float4 f = xp[v ^ (gc & 7)];
              x[m][4 * v + 0] = f.x;
              x[m][4 * v + 1] = f.y;
              x[m][4 * v + 2] = f.z;
              x[m][4 * v + 3] = f.w;
            }
          }
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            float d[MT];
            group_dot16_rows<MT>(x, w[j][i], d);
            const float sv = valid ? s[j][i] : 0.0f;
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][i] = fmaf(sv, d[m] * 0.0625f, acc[m][i]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[m][i] = segment_sum<64>(acc[m][i]);
      if (lane == 63) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const int n = n0 + i;
            if (m0 + m < me && n < n_end) Y[long(r0 + m0 + m) * N + n] = acc[m][i];
          }
      }
    }
  }
}


// ------------------------------------------------------------ matrix cores
//
// grouped_mfma<MR, kSrc, kOnePass>: the same product on v_mfma_f32_16x16x32_f16, with
// the split path's arithmetic: exact weight codes q - 8, two fp16 limbs of
// each prescaled activation, fp32 accumulation, one fp32 FMA per group for
// the scale, the row's power of two undone at the store.  Rows 0..MR-1 of the
// 16-row MFMA tile carry up to MR slots of one expert; the other rows are
// zero, so each weight is converted once and met by all the slots in one
// instruction instead of one FMA per slot.
//
// A workgroup of kMfmaWaves waves takes work items: (expert, chunk of up to
// MR of the expert's slots, block of kMfmaCols = 16 x kMfmaWaves columns).
//  * staging: the chunk's token rows are read (once, before the weight loads,
//    when they fit in registers) for each row's maximum, i.e. its
//    power-of-two exponent, and split into LDS as MFMA A fragments: 16-byte
//    chunk (g*4 + b)*MR + r holds the 8 limbs of k block b of group g of slot
//    r; hi region, then lo region, each followed by a zero region of 4 groups
//    that steps past the last group read.  Tile rows past the chunk's slots
//    read slot rows too: they only make output rows that are never stored.
//  * each wave streams its 16 weight rows.  Lane (c, R), R the lane's 16-lane
//    row, loads the 16 bytes of group 4s + R of weight row c, so one load
//    covers 4 groups of 16 rows with 64 contiguous bytes per row.  Two rounds
//    of lane swaps across the four 16-lane rows transpose that to word R of
//    each of the 4 groups in lane (c, R): the MFMA's B operand.  Per group:
//    hi and lo MFMAs into one zeroed tile, then one FMA per slot row with the
//    group's scale.  Loads run kMfmaPD steps ahead.
//  * the staging barriers wait for LDS traffic only, never for the weight
//    loads in flight.
//  * slot rows 0..MR-1 of the result tile sit in lanes 0..15 (column c, 4
//    rows each), which write Y.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kMfmaCols = 16 * kMfmaWaves;
constexpr int kMfmaPD = 8;                 // 4-group steps in flight per wave
// Where a wave's weights and scales come from: the public layout with one
// 16-byte scale load per step (G % 4 == 0), the public layout with four
// scale loads (G % 4 != 0), or the packed layout of w4a16_grouped_pack.
constexpr int kSrcPublic = 0;
constexpr int kSrcPublicScalar = 1;
constexpr int kSrcPacked = 2;

// the ring depth: shallower when the scales take four loads, to stay within
// the registers of 8 waves per compute unit
template <int kSrc>
constexpr int kMfmaDepth = kSrc == kSrcPublicScalar ? kMfmaPD - 2 : kMfmaPD;
constexpr int kMfmaMaxLds = 150 * 1024;

// bytes of one limb region for MR rows and G4 groups (with its zero region of
// 4 groups), and of the whole LDS image (without the work list)
__host__ __device__ constexpr int mfma_region_bytes(int MR, int G4) { return (G4 + 4) * 4 * MR * 16; }

__host__ __device__ constexpr int mfma_lds_bytes(int MR, int G4) {
  return 2 * mfma_region_bytes(MR, G4) + kMfmaWaves * MR * 4;
}

// LDS writes of this wave complete, then the workgroup barrier; the wave's
// global loads stay in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// max |x| over one 8-wide block held as two float4
__device__ __forceinline__ float block_absmax(float4 a, float4 c) {
  return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
               fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
}

// one 4-group step of weights and the 4 scales of the lane's row.  Public
// layout: lane (c, R) loads group 4*step + R of its row (wrow, srow: the
// row); packed layout: the lane's 16 bytes of the tile's step block, already
// word R of each of the 4 groups (wrow: the tile's first block plus the lane;
// srow: the tile's first scale block plus 4 c)
template <int kSrc>
__device__ __forceinline__ void mfma_load_w(const uint4 *__restrict__ wrow, int G, int step, int R,
                                            uint4 &w) {
  if constexpr (kSrc == kSrcPacked) {
    w = load_stream16(wrow + long(step) * 64);
  } else {
    w = load_stream16(wrow + std::min(4 * step + R, G - 1));
  }
}

template <int kSrc>
__device__ __forceinline__ void mfma_load_s(const float *__restrict__ srow, int G, int step,
                                            float4 &s) {
  if constexpr (kSrc == kSrcPacked) {
    s = *reinterpret_cast<const float4 *>(srow + long(step) * 64);
  } else if constexpr (kSrc == kSrcPublic) {
    s = *reinterpret_cast<const float4 *>(srow + 4 * step);
  } else {
    s.x = srow[std::min(4 * step + 0, G - 1)];
    s.y = srow[std::min(4 * step + 1, G - 1)];
    s.z = srow[std::min(4 * step + 2, G - 1)];
    s.w = srow[std::min(4 * step + 3, G - 1)];
  }
}

template <int kSrc>
__device__ __forceinline__ void mfma_load(const uint4 *__restrict__ wrow,
                                          const float *__restrict__ srow, int G, int step, int R,
                                          uint4 &w, float4 &s) {
  mfma_load_w<kSrc>(wrow, G, step, R, w);
  mfma_load_s<kSrc>(srow, G, step, s);
}

// lane row R holds words 0..3 of group R; afterwards word R of groups 0..3
// (v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 of its second; v_permlane16_swap the odd 16-lane rows of the
// first with the even rows of the second)
__device__ __forceinline__ void transpose4(uint32_t &v0, uint32_t &v1, uint32_t &v2,
                                           uint32_t &v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v0 = c[0];
  v1 = c[1];
  v2 = d[0];
  v3 = d[1];
}

// one 4-group step: operand reads, weight conversion, reload of the ring
// slot kMfmaPD steps ahead (pinned right after the slot's last use of the
// weights; the scales after the FMAs), MFMAs and scale FMAs.  kLive: the step
// is below S and its reload in range (no clamps, no selects); otherwise a
// step at or past S reads the zero chunk and adds exactly 0, and the reload
// is clamped to the last step.
template <int MR, int MC, int kSrc>
__device__ __forceinline__ void mfma_step(const unsigned char *__restrict__ xa, int a_off,
                                          int reg, int zregion, const uint4 *__restrict__ wrow,
                                          const float *__restrict__ srow, int G, int S, int step,
                                          int R, uint4 &w, float4 &s, float (&acc)[4]) {
  constexpr int AG = 4 * MR * 16;  // bytes between consecutive groups' A fragments
  constexpr int PD = kMfmaDepth<kSrc>;
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int next = std::min(step + PD, S - 1);
  // a step at or past S reads the zero region (4 groups of zero fragments,
  // same stride) and adds exactly 0
  const unsigned char *ap = xa + (step < S ? a_off + 4 * step * AG : zregion);
  half8_t ah[4], al[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ah[q] = *reinterpret_cast<const half8_t *>(ap + q * AG);
    al[q] = *reinterpret_cast<const half8_t *>(ap + q * AG + reg);
  }
  uint32_t v0 = w.x, v1 = w.y, v2 = w.z, v3 = w.w;
  if constexpr (kSrc != kSrcPacked) transpose4(v0, v1, v2, v3);
  const half8_t b0 = nibbles_to_f16(v0), b1 = nibbles_to_f16(v1);
  const half8_t b2 = nibbles_to_f16(v2), b3 = nibbles_to_f16(v3);
  __builtin_amdgcn_sched_barrier(0);
  mfma_load_w<kSrc>(wrow, G, next, R, w);
  __builtin_amdgcn_sched_barrier(0);
  // the 4 groups are independent: hi MFMAs, lo MFMAs, then the scales
  floatx4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[0], b0, zero, 0, 0, 0);
  floatx4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[1], b1, zero, 0, 0, 0);
  floatx4 d2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[2], b2, zero, 0, 0, 0);
  floatx4 d3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[3], b3, zero, 0, 0, 0);
  d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[0], b0, d0, 0, 0, 0);
  d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[1], b1, d1, 0, 0, 0);
  d2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[2], b2, d2, 0, 0, 0);
  d3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[3], b3, d3, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    acc[i] = fmaf(s.x, d0[i], acc[i]);
    acc[i] = fmaf(s.y, d1[i], acc[i]);
    acc[i] = fmaf(s.z, d2[i], acc[i]);
    acc[i] = fmaf(s.w, d3[i], acc[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_load_s<kSrc>(srow, G, next, s);
  __builtin_amdgcn_sched_barrier(0);
}

// the wave's 16 columns over all S steps for MC slot rows.  w/s form a ring
// of PD 4-group steps holding steps 0..PD-1 on entry; each step reloads its
// slot PD steps ahead, right after the slot's last use, so the ring keeps its
// registers across the loop's back edge and a step waits only for its own
// loads (a reload moved later, or a copy of a value still in flight, would
// make a step wait for all loads).  The loop runs whole rings, the steps past
// S adding 0, so it has no branch inside.
template <int MR, int MC, int kSrc, int PD>
__device__ __forceinline__ void mfma_stream(const unsigned char *__restrict__ xa, int a_off,
                                            int reg, int zregion, const uint4 *__restrict__ wrow,
                                            const float *__restrict__ srow, int G, int S,
                                            uint4 (&w)[PD], float4 (&s)[PD], float (&acc)[4]) {
  static_assert(PD == kMfmaDepth<kSrc>, "ring depth");
  const int R = (threadIdx.x & 63) >> 4;
  for (int s0 = 0; s0 < S; s0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p)
      mfma_step<MR, MC, kSrc>(xa, a_off, reg, zregion, wrow, srow, G, S, s0 + p, R, w[p], s[p],
                              acc);
  }
}

// one chunk of MC (<= MR) slots: row maxima, the limb split, the stream.
template <int MR, int MC, int kSrc, bool kOnePass>
__device__ __forceinline__ void mfma_chunk(const float *__restrict__ X,
                                           const int32_t *__restrict__ token_index,
                                           unsigned char *__restrict__ xa, float *__restrict__ red,
                                           float *__restrict__ Y, int T, int N, int G, int rbase, int n0, const uint4 *__restrict__ wrow,
                                           const float *__restrict__ srow) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int G4 = (G + 3) & ~3;
  const int K8 = G * 4;
  const int S = G4 / 4;
  const int reg = mfma_region_bytes(MR, G4);
  const int zregion = G4 * 4 * MR * 16;
  const float4 *X4 = reinterpret_cast<const float4 *>(X);
  const long K4 = long(K8) * 2;
  const int R_ = lane >> 4;
  constexpr int PD = kMfmaDepth<kSrc>;

  long xrow[MC];  // float4 offset of each slot's token row
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    const int tok = token_index[rbase + r];
    xrow[r] = long(std::min(std::max(tok, 0), T - 1)) * K4;
  }
  // kOnePass (4 G4 <= 2 kMfmaThreads 8-wide blocks per row): the token rows
  // are read once, before the weights, and kept in registers for the split
  float4 a[MC][2], c[MC][2];
  if constexpr (kOnePass) {
#pragma unroll
    for (int r = 0; r < MC; ++r)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const long j = std::min(t + u * kMfmaThreads, K8 - 1);
        a[r][u] = X4[xrow[r] + 2 * j];
        c[r][u] = X4[xrow[r] + 2 * j + 1];
      }
  }
  // the ring's first weight loads: they do not depend on the activations
  // (waves past N load clamped rows and compute with them, but store nothing)
  uint4 w[PD];
  float4 s[PD];
#pragma unroll
  for (int p = 0; p < PD; ++p) mfma_load<kSrc>(wrow, srow, G, std::min(p, S - 1), R_, w[p], s[p]);

  // row maxima
  float mx[MC];
#pragma unroll
  for (int r = 0; r < MC; ++r) mx[r] = 0.0f;
  if constexpr (kOnePass) {
#pragma unroll
    for (int r = 0; r < MC; ++r)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        mx[r] = fmaxf(mx[r], block_absmax(a[r][u], c[r][u]));
  } else {
    for (int j0 = t; j0 < K8; j0 += 2 * kMfmaThreads) {
      float4 a2[MC][2], c2[MC][2];
#pragma unroll
      for (int r = 0; r < MC; ++r)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const long j = std::min(j0 + u * kMfmaThreads, K8 - 1);
          a2[r][u] = X4[xrow[r] + 2 * j];
          c2[r][u] = X4[xrow[r] + 2 * j + 1];
        }
#pragma unroll
      for (int r = 0; r < MC; ++r)
#pragma unroll
        for (int u = 0; u < 2; ++u) mx[r] = fmaxf(mx[r], block_absmax(a2[r][u], c2[r][u]));
    }
  }
  lds_barrier();  // the previous chunk's limbs and maxima are no longer read
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    float v = mx[r];
    for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
    if (lane == 0) red[wave * MR + r] = v;
  }
  lds_barrier();
  int ex[MC];
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < kMfmaWaves; ++q) v = fmaxf(v, red[q * MR + r]);
    ex[r] = row_exponent(v);
  }

  // the split into the A-fragment layout; blocks of groups past G are zero
  for (int j0 = t; j0 < 4 * G4; j0 += 2 * kMfmaThreads) {
    if constexpr (!kOnePass) {
#pragma unroll
      for (int r = 0; r < MC; ++r)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const long j = std::min(j0 + u * kMfmaThreads, K8 - 1);
          a[r][u] = X4[xrow[r] + 2 * j];
          c[r][u] = X4[xrow[r] + 2 * j + 1];
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + u * kMfmaThreads;
      if (j < 4 * G4) {
#pragma unroll
        for (int r = 0; r < MC; ++r) {
          half8_t h, l;
          if (j < K8) {
            split_block(a[r][u], c[r][u], ex[r], h, l);
          } else {
            h = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
            l = h;
          }
          *reinterpret_cast<half8_t *>(xa + (j * MR + r) * 16) = h;
          *reinterpret_cast<half8_t *>(xa + reg + (j * MR + r) * 16) = l;
        }
      }
    }
  }
  lds_barrier();

  // tile rows past MC read slot rows of the chunk as well: they only make
  // output rows that are never stored, and every lane keeps one stride
  const int a_off = (R_ * MR + std::min(lane & 15, MC - 1)) * 16;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // the ring's first loads (issued before the staging) are in by now; with
  // nothing in flight on entry, the waits inside the stream's loop stay exact
  // (each step waits for its own loads only) instead of draining every ring
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  mfma_stream<MR, MC, kSrc, PD>(xa, a_off, reg, zregion, wrow, srow, G, S, w, s, acc);
  const int n = n0 + lane;
  if (n0 < N && lane < 16 && n < N) {
#pragma unroll
    for (int i = 0; i < MC; ++i) Y[long(rbase + i) * N + n] = ldexpf(acc[i], -ex[i]);
  }
}

// A persistent grid (one workgroup per compute unit, fewer when there is
// less work) walks a list of equal work items: (expert, chunk of MR slots,
// block of kMfmaCols columns), only those that exist.  Each workgroup turns
// the expert offsets into a prefix sum of chunks per expert in LDS and takes
// items blockIdx.x, blockIdx.x + gridDim.x, ...; an item's expert is found by
// binary search.  (Launching a workgroup per possible item instead leaves
// most of them empty, and workgroups that leave at once still hold back the
// dispatch of those behind them.)  Every workgroup leaves when its next item
// index passes the item count.
constexpr int kMfmaMaxExperts = 4096;

template <int MR, int kSrc, bool kOnePass>
__global__ void __launch_bounds__(kMfmaThreads)
grouped_mfma(const float *__restrict__ X, const int32_t *__restrict__ token_index,
             const int32_t *__restrict__ offsets, const uint4 *__restrict__ qw,
             const float *__restrict__ sc, float *__restrict__ Y, int T, int R, int E, int N,
             int G) {
  extern __shared__ __align__(16) unsigned char xa[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int G4 = (G + 3) & ~3;
  const int reg = mfma_region_bytes(MR, G4);
  float *red = reinterpret_cast<float *>(xa + 2 * reg);
  int *pre = reinterpret_cast<int *>(xa + 2 * reg + kMfmaWaves * MR * 4);  // [E + 1]
  int *part = pre + E + 1;                                                  // [kMfmaThreads]
  const int n_blocks = (N + kMfmaCols - 1) / kMfmaCols;

  // chunks per expert, then their prefix sum: with E <= 64 one wave's
  // shuffle scan; otherwise a serial one over each thread's run of experts
  // and an inclusive scan of the runs' totals
  if (E <= 64) {
    if (t < 64) {
      int cnt = 0;
      if (t < E) {
        const int r0 = std::min(std::max(offsets[t], 0), R);
        const int r1 = std::min(std::max(offsets[t + 1], r0), R);
        cnt = (r1 - r0 + MR - 1) / MR;
      }
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(cnt, d);
        if (t >= d) cnt += v;
      }
      if (t < E) pre[t + 1] = cnt;
      if (t == 0) pre[0] = 0;
    }
  } else {
  const int per = (E + kMfmaThreads - 1) / kMfmaThreads;
  const int e_lo = std::min(E, t * per), e_hi = std::min(E, e_lo + per);
  int run = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    const int r0 = std::min(std::max(offsets[e], 0), R);
    const int r1 = std::min(std::max(offsets[e + 1], r0), R);
    run += (r1 - r0 + MR - 1) / MR;
    pre[e + 1] = run;  // within the run, completed below
  }
  part[t] = run;
  __syncthreads();
  for (int d = 1; d < kMfmaThreads; d <<= 1) {
    const int v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const int base = t > 0 ? part[t - 1] : 0;
  for (int e = e_lo; e < e_hi; ++e) pre[e + 1] += base;
  if (t == 0) pre[0] = 0;
  }
  // the zero regions after each limb region (never overwritten; the barrier
  // below orders these stores before any read)
  for (int i = t; i < 4 * 4 * MR; i += kMfmaThreads) {
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    *reinterpret_cast<float4 *>(xa + G4 * 4 * MR * 16 + i * 16) = z4;
    *reinterpret_cast<float4 *>(xa + reg + G4 * 4 * MR * 16 + i * 16) = z4;
  }
  __syncthreads();

  const long items = long(pre[E]) * n_blocks;
  for (long i = blockIdx.x; i < items; i += gridDim.x) {
    const int k = int(i / n_blocks);
    const int cb = int(i - long(k) * n_blocks);
    int lo = 0, hi = E;  // the expert e with pre[e] <= k < pre[e + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= k) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int r0 = std::min(std::max(offsets[e], 0), R);
    const int r1 = std::min(std::max(offsets[e + 1], r0), R);
    const int m0 = (k - pre[e]) * MR;
    const int mc = std::min(MR, r1 - r0 - m0);
    const int rbase = r0 + m0;
    const int n0 = cb * kMfmaCols + (t >> 6) * 16;
    const uint4 *wrow;
    const float *srow;
    if constexpr (kSrc == kSrcPacked) {
      // the wave's 16-row tile (clamped: waves past N compute but store nothing)
      const long tiles = (N + 15) / 16;
      const long tile = long(e) * tiles + std::min(long(n0 / 16), tiles - 1);
      const long S4 = (G + 3) / 4;
      wrow = qw + tile * S4 * 64 + lane;
      srow = sc + (tile * S4 * 16 + (lane & 15)) * 4;
    } else {
      const long nrow = std::min(n0 + (lane & 15), N - 1);
      wrow = qw + (long(e) * N + nrow) * G;
      srow = sc + (long(e) * N + nrow) * G;
    }
    switch (mc) {
      case 1: mfma_chunk<MR, 1, kSrc, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow); break;
      case 2:
        if constexpr (MR >= 2) mfma_chunk<MR, 2, kSrc, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
        break;
      case 3:
        if constexpr (MR >= 4) mfma_chunk<MR, 3, kSrc, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
        break;
      default:
        if constexpr (MR >= 4) mfma_chunk<MR, 4, kSrc, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
        break;
    }
  }
}

struct MfmaPlan {
  int MR, grid;
  size_t lds;
};

// MR from the mean slots per active expert (an expert with more slots makes
// more chunks), fewer rows when all of K does not fit the LDS budget; the
// grid is one workgroup per compute unit, or the most items there can be.
bool plan_mfma(int T, int R, int E, int N, int G, int cus, MfmaPlan &p) {
  (void)T;
  if (E > kMfmaMaxExperts) return false;
  const int active = std::max(1, std::min(E, R));
  const double mean = double(R) / active;
  p.MR = mean <= 1.0 ? 1 : (mean <= 1.5 ? 2 : 4);
  const int G4 = (G + 3) & ~3;
  auto lds = [&](int mr) {
    return size_t(mfma_lds_bytes(mr, G4)) + size_t(E + 1 + kMfmaThreads) * 4;
  };
  while (lds(p.MR) > size_t(kMfmaMaxLds)) {
    if (p.MR == 1) return false;
    p.MR /= 2;
  }
  p.lds = lds(p.MR);
  const long n_blocks = (N + kMfmaCols - 1) / kMfmaCols;
  const long max_items = n_blocks * (long(R + p.MR - 1) / p.MR + active);
  p.grid = int(std::max(1L, std::min(long(std::max(cus, 1)), max_items)));
  return true;
}

template <int MR>
hipError_t run_mfma(const MfmaPlan &p, const float *X, const int32_t *token_index,
                    const int32_t *offsets, const uint4 *qw, const float *sc, bool packed,
                    float *Y, int T, int R, int E, int N, int G, hipStream_t stream) {
  const bool one_pass = 4 * ((G + 3) & ~3) <= 2 * kMfmaThreads;
  const int src = packed ? kSrcPacked : (G % 4 == 0 ? kSrcPublic : kSrcPublicScalar);
#define W4A16_GROUPED_MFMA(SRC, ONE)                                                             \
  hipLaunchKernelGGL((grouped_mfma<MR, SRC, ONE>), dim3(p.grid), dim3(kMfmaThreads), p.lds,      \
                     stream, X, token_index, offsets, qw, sc, Y, T, R, E, N, G)
  switch (src * 2 + (one_pass ? 1 : 0)) {
    case kSrcPublic * 2 + 1: W4A16_GROUPED_MFMA(kSrcPublic, true); break;
    case kSrcPublic * 2: W4A16_GROUPED_MFMA(kSrcPublic, false); break;
    case kSrcPublicScalar * 2 + 1: W4A16_GROUPED_MFMA(kSrcPublicScalar, true); break;
    case kSrcPublicScalar * 2: W4A16_GROUPED_MFMA(kSrcPublicScalar, false); break;
    case kSrcPacked * 2 + 1: W4A16_GROUPED_MFMA(kSrcPacked, true); break;
    default: W4A16_GROUPED_MFMA(kSrcPacked, false); break;
  }
#undef W4A16_GROUPED_MFMA
  return hipGetLastError();
}

hipError_t run_mfma_any(const MfmaPlan &p, const float *X, const int32_t *token_index,
                        const int32_t *offsets, const uint4 *qw, const float *sc, bool packed,
                        float *Y, int T, int R, int E, int N, int G, hipStream_t stream) {
  switch (p.MR) {
    case 1: return run_mfma<1>(p, X, token_index, offsets, qw, sc, packed, Y, T, R, E, N, G, stream);
    case 2: return run_mfma<2>(p, X, token_index, offsets, qw, sc, packed, Y, T, R, E, N, G, stream);
    default: return run_mfma<4>(p, X, token_index, offsets, qw, sc, packed, Y, T, R, E, N, G, stream);
  }
}

// ------------------------------------------------------------ repack
//
// The packed layout of w4a16_grouped_pack: for expert e, 16-row tile t
// (T16 = ceil(N/16) tiles) and 4-group step s (S4 = ceil(G/4) steps), block
// b = (e*T16 + t)*S4 + s holds
//  * 64 chunks of 16 bytes at b*64 + l: for lane l = c + 16 R, word R of
//    groups 4s, 4s+1, 4s+2, 4s+3 of row 16t + c (the MFMA B operand after
//    the lane transpose of the public layout);
//  * after all weight blocks, 16 x 4 scales at float (b*16 + c)*4 + q: the
//    scale of group 4s + q of row 16t + c.
// Rows past N and groups past G hold the word 0x88888888 (every code 8, so
// weight 0) and scale 0.  One thread per 16-byte chunk; bits are moved only.
__global__ void __launch_bounds__(256)
grouped_pack(const uint32_t *__restrict__ qw, const float *__restrict__ sc, uint4 *__restrict__ pw,
             float4 *__restrict__ ps, int N, int G, long blocks) {
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  const long T16 = (N + 15) / 16, S4 = (G + 3) / 4;
  if (i < blocks * 64) {  // a weight chunk
    const long b = i / 64;
    const int l = int(i - b * 64), c = l & 15, R = l >> 4;
    const long s4 = b % S4, et = b / S4;
    const long t = et % T16, e = et / T16;
    const long n = t * 16 + c;
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long g = s4 * 4 + q;
      v[q] = (n < N && g < G) ? qw[((e * N + n) * G + g) * 4 + R] : 0x88888888u;
    }
    pw[i] = make_uint4(v[0], v[1], v[2], v[3]);
  } else if (i < blocks * 64 + blocks * 16) {  // a scale chunk
    const long j = i - blocks * 64;
    const long b = j / 16;
    const int c = int(j - b * 16);
    const long s4 = b % S4, et = b / S4;
    const long t = et % T16, e = et / T16;
    const long n = t * 16 + c;
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const long g = s4 * 4 + q;
      v[q] = (n < N && g < G) ? sc[(e * N + n) * G + g] : 0.0f;
    }
    ps[j] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

long grouped_pack_blocks(int E, int N, int G) {
  return long(E) * ((N + 15) / 16) * ((G + 3) / 4);
}

struct RowsPlan {
  int MT, RB, rows_per_block, blocks;
  size_t lds;
};

// MT from the mean slots per expert; about 2048 row blocks over the experts
// that can be active (at most min(E, R)), down to one chunk of RB rows per
// wave: an expert with many slots makes several passes over its rows, and
// spreading its rows over many blocks keeps that pass count from becoming the
// launch's long pole.
bool plan_rows(int R, int E, int N, int G, RowsPlan &p) {
  const int active = std::max(1, std::min(E, R));
  const int mean = (R + active - 1) / active;
  p.MT = mean >= 3 ? 4 : (mean == 2 ? 2 : 1);
  p.RB = p.MT == 4 ? 2 : 4;
  p.lds = size_t(p.MT) * G * kGroup * sizeof(float);
  if (p.lds > size_t(kRowsMaxLds)) return false;
  const int max_blocks = std::max(1, (N + 4 * p.RB - 1) / (4 * p.RB));
  const int per_expert = std::min(max_blocks, std::max(1, (2048 + active - 1) / active));
  p.rows_per_block = (N + per_expert - 1) / per_expert;
  p.blocks = (N + p.rows_per_block - 1) / p.rows_per_block;
  return true;
}

template <int MT, int RB>
hipError_t run_rows(const RowsPlan &p, const float *X, const int32_t *token_index,
                    const int32_t *offsets, const int32_t *qw, const float *sc, float *Y, int T,
                    int R, int E, int N, int G, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_rows<MT, RB>), dim3(p.blocks, E), dim3(kRowsThreads), p.lds, stream,
                     X, token_index, offsets, reinterpret_cast<const uint4 *>(qw), sc, Y, T, R, N,
                     G, p.rows_per_block);
  return hipGetLastError();
}

struct GroupedPlan {
  int TPS, S, BS, RB, MT, TR, blocks;
};

int floor_pow2(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

// MT from the mean number of slots per expert; RB so that the active experts'
// blocks keep about 256 CUs x 7 waves of 16-byte loads in flight; S the slot
// count with the fewest idle lanes in whole waves.
GroupedPlan plan_grouped(int R, int E, int N, int G) {
  GroupedPlan p;
  p.TPS = std::min(G, kMaxBlockG);
  const int mean = (R + E - 1) / E;
  p.MT = mean >= 3 ? 4 : (mean == 2 ? 2 : 1);
  const long active = std::min(E, R);
  const long chunks = long(N) * p.TPS * active;
  p.RB = 8 / p.MT;
  while (p.RB > 1 && chunks / p.RB < 256L * 7 * 64) p.RB /= 2;
  int best_s = 1, best_idle = 1 << 30;
  for (int s = 1; s * p.TPS <= kMaxBlockG; ++s) {
    const int bs = ((s * p.TPS + 63) / 64) * 64;
    const int idle = (bs - s * p.TPS) * 1024 / bs;
    if (idle < best_idle) {
      best_idle = idle;
      best_s = s;
    }
  }
  p.S = best_s;
  p.BS = ((p.S * p.TPS + 63) / 64) * 64;
  p.blocks = int((long(N) + long(p.S) * p.RB - 1) / (long(p.S) * p.RB));
  p.TR = std::min(64, std::max(1, floor_pow2(std::max(1, p.BS / (p.MT * p.S * p.RB)))));
  return p;
}

template <int MT, int RB>
hipError_t run_grouped(const GroupedPlan &p, const float *X, const int32_t *token_index,
                       const int32_t *offsets, const int32_t *qw, const float *sc, float *Y,
                       int T, int R, int E, int N, int G, hipStream_t stream) {
  const size_t lds = size_t(MT) * RB * (p.BS + 1) * sizeof(float);
  hipLaunchKernelGGL((gemv_grouped<MT, RB>), dim3(p.blocks, E), dim3(p.BS), lds, stream, X,
                     token_index, offsets, reinterpret_cast<const uint4 *>(qw), sc, Y, T, R, N,
                     G, p.S, p.TPS, p.TR);
  return hipGetLastError();
}

}  // namespace

// compute units of the current device (queried once per device)
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int grouped_kernel(int T, int R, int E, int N, int K) {
  const int G = K / kGroup;
  MfmaPlan mp;
  if (plan_mfma(T, R, E, N, G, 256, mp)) return 1;  // the choice does not depend on the CU count
  RowsPlan rp;
  if (plan_rows(R, E, N, G, rp)) return 2;
  return 3;
}

hipError_t launch_grouped(const float *X, const int32_t *token_index, const int32_t *offsets,
                          const int32_t *qweight, const float *scales, float *Y, int T, int R,
                          int E, int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  if (E > 65535) return hipErrorInvalidConfiguration;
  MfmaPlan mp;
  const int cus = compute_units();
  if (plan_mfma(T, R, E, N, G, cus, mp))
    return run_mfma_any(mp, X, token_index, offsets, reinterpret_cast<const uint4 *>(qweight),
                        scales, false, Y, T, R, E, N, G, stream);
  RowsPlan rp;
  if (plan_rows(R, E, N, G, rp)) {
    switch (rp.MT) {
      case 1: return run_rows<1, 4>(rp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
      case 2: return run_rows<2, 4>(rp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
      default: return run_rows<4, 2>(rp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    }
  }
  const GroupedPlan p = plan_grouped(R, E, N, G);
  switch (p.MT * 16 + p.RB) {
    case 1 * 16 + 8: return run_grouped<1, 8>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 1 * 16 + 4: return run_grouped<1, 4>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 1 * 16 + 2: return run_grouped<1, 2>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 1 * 16 + 1: return run_grouped<1, 1>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 2 * 16 + 4: return run_grouped<2, 4>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 2 * 16 + 2: return run_grouped<2, 2>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 2 * 16 + 1: return run_grouped<2, 1>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 4 * 16 + 2: return run_grouped<4, 2>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    case 4 * 16 + 1: return run_grouped<4, 1>(p, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t grouped_pack_bytes(int E, int N, int K) {
  return size_t(grouped_pack_blocks(E, N, K / kGroup)) * (1024 + 256);
}

hipError_t launch_grouped_pack(const int32_t *qweight, const float *scales, void *packed, int E,
                               int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  const long blocks = grouped_pack_blocks(E, N, G);
  const long chunks = blocks * (64 + 16);
  if ((chunks + 255) / 256 > 0x7fffffffL) return hipErrorInvalidConfiguration;
  uint4 *pw = static_cast<uint4 *>(packed);
  float4 *ps = reinterpret_cast<float4 *>(pw + blocks * 64);
  hipLaunchKernelGGL(grouped_pack, dim3(unsigned((chunks + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t *>(qweight), scales, pw, ps, N, G, blocks);
  return hipGetLastError();
}

bool grouped_packed_supported(int T, int R, int E, int N, int K) {
  MfmaPlan mp;
  return plan_mfma(T, R, E, N, K / kGroup, 256, mp);
}

hipError_t launch_grouped_packed(const float *X, const int32_t *token_index,
                                 const int32_t *offsets, const void *packed, float *Y, int T,
                                 int R, int E, int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  if (E > 65535) return hipErrorInvalidConfiguration;
  MfmaPlan mp;
  if (!plan_mfma(T, R, E, N, G, compute_units(), mp)) return hipErrorInvalidValue;
  const long blocks = grouped_pack_blocks(E, N, G);
  const uint4 *pw = static_cast<const uint4 *>(packed);
  const float *ps = reinterpret_cast<const float *>(pw + blocks * 64);
  return run_mfma_any(mp, X, token_index, offsets, pw, ps, true, Y, T, R, E, N, G, stream);
}

}  // namespace w4a16
