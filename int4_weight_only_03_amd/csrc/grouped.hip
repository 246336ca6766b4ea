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
// grouped_mfma<MR, kSc4>: the same product on v_mfma_f32_16x16x32_f16, with
// the split path's arithmetic: exact weight codes q - 8, two fp16 limbs of
// each prescaled activation, fp32 accumulation, one fp32 FMA per group for
// the scale, the row's power of two undone at the store.  Rows 0..MR-1 of the
// 16-row MFMA tile carry up to MR slots of one expert; the other rows are
// zero, so each weight is converted once and met by all the slots in one
// instruction instead of one FMA per slot.
//
// A workgroup of kMfmaWaves waves serves one expert, kMfmaCols consecutive
// output columns (16 per wave) and one chunk of MR of the expert's slots
// (chunks c0, c0 + C, ... of that expert):
//  * the chunk's token rows are read once for each row's maximum (its
//    power-of-two exponent), then K is taken in windows of W groups: the
//    window's limbs are split into LDS as MFMA A fragments (16-byte chunk
//    ((g - w0)*4 + b)*MR + r holds the 8 limbs of k block b of group g of
//    slot r; hi region, then lo region, each ending with a zero chunk that the
//    tile rows past the chunk's slots read) and the waves stream that window.
//    Windows keep the workgroup's LDS under 64 KB: larger allocations left
//    many compute units unable to take a workgroup.
//  * each wave streams its 16 weight rows.  Lane (c, R), R the lane's 16-lane
//    row, loads the 16 bytes of group 4s + R of weight row c, so one load
//    covers 4 groups of 16 rows with 64 contiguous bytes per row.  Two rounds
//    of lane swaps across the four 16-lane rows transpose that to word R of
//    each of the 4 groups in lane (c, R): the MFMA's B operand.  Per group:
//    hi and lo MFMAs into one zeroed tile, then one FMA per slot row with the
//    group's scale.  Loads run kMfmaPD steps ahead, across windows.
//  * the barriers between phases wait for LDS traffic only, never for the
//    weight loads in flight.
//  * slot rows 0..MR-1 of the result tile sit in lanes 0..15 (column c, 4
//    rows each), which write Y.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaThreads = 64 * kMfmaWaves;
constexpr int kMfmaCols = 16 * kMfmaWaves;
constexpr int kMfmaPD = 8;                 // 4-group steps in flight per wave
// the ring depth: shallower when the scales take four loads (G % 4 != 0), to
// stay within the registers of 8 waves per compute unit
template <bool kSc4>
constexpr int kMfmaDepth = kSc4 ? kMfmaPD : kMfmaPD - 2;
constexpr int kMfmaMaxLds = 150 * 1024;

// bytes of one limb region for MR rows and a window of W groups (with its
// zero chunk), and of the whole LDS image
__host__ __device__ constexpr int mfma_region_bytes(int MR, int G4) { return G4 * 4 * MR * 16 + 16; }

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

// one 4-group step of weights (lane (c, R): group 4*step + R of its row) and
// the 4 scales of its row
template <bool kSc4>
__device__ __forceinline__ void mfma_load(const uint4 *__restrict__ wrow,
                                          const float *__restrict__ srow, int G, int step, int R,
                                          uint4 &w, float4 &s) {
  w = load_stream16(wrow + std::min(4 * step + R, G - 1));
  if constexpr (kSc4) {
    s = *reinterpret_cast<const float4 *>(srow + 4 * step);
  } else {
    s.x = srow[std::min(4 * step + 0, G - 1)];
    s.y = srow[std::min(4 * step + 1, G - 1)];
    s.z = srow[std::min(4 * step + 2, G - 1)];
    s.w = srow[std::min(4 * step + 3, G - 1)];
  }
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

// steps [s_begin, s_end) of the wave's 16 columns for MC slot rows, s_begin a
// multiple of kMfmaPD.  w/s form a ring of kMfmaPD 4-group steps holding
// steps s_begin.. on entry; each step reloads its slot kMfmaPD steps ahead:
// the weights once they are converted, the scales once the FMAs have used
// them.  Each reload follows the last use of the slot's old value and is
// pinned there, so the ring keeps its registers across the loop's back edge
// and a step waits only for its own loads (a reload moved later, or a copy of
// a value still in flight, would make a step wait for all loads).  Steps at
// or past S read the zero chunk and add exactly 0, so the ring's steps run
// without branches.  LDS group offsets are relative to the window's first
// group, 4 * s_begin.
template <int MC, bool kSc4, int PD>
__device__ __forceinline__ void mfma_stream(const unsigned char *__restrict__ xa, int a_off,
                                            int a_g, int reg, int zchunk,
                                            const uint4 *__restrict__ wrow,
                                            const float *__restrict__ srow, int G, int S,
                                            int s_begin, int s_end, uint4 (&w)[PD],
                                            float4 (&s)[PD], float (&acc)[4]) {
  const int R = (threadIdx.x & 63) >> 4;
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = s_begin; s0 < s_end; s0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int step = s0 + p;
      const int next = std::min(step + PD, S - 1);
      const bool live = step < S;
      // operand reads for the 4 groups, then the weight conversions
      const int ag = live ? a_g : 0;
      const unsigned char *ap = xa + (live ? a_off + 4 * (step - s_begin) * a_g : zchunk);
      half8_t ah[4], al[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ah[q] = *reinterpret_cast<const half8_t *>(ap + q * ag);
        al[q] = *reinterpret_cast<const half8_t *>(ap + q * ag + reg);
      }
      uint32_t v0 = w[p].x, v1 = w[p].y, v2 = w[p].z, v3 = w[p].w;
      transpose4(v0, v1, v2, v3);
      const half8_t b0 = nibbles_to_f16(v0), b1 = nibbles_to_f16(v1);
      const half8_t b2 = nibbles_to_f16(v2), b3 = nibbles_to_f16(v3);
      __builtin_amdgcn_sched_barrier(0);
      w[p] = load_stream16(wrow + std::min(4 * next + R, G - 1));
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
        acc[i] = fmaf(s[p].x, d0[i], acc[i]);
        acc[i] = fmaf(s[p].y, d1[i], acc[i]);
        acc[i] = fmaf(s[p].z, d2[i], acc[i]);
        acc[i] = fmaf(s[p].w, d3[i], acc[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSc4) {
        s[p] = *reinterpret_cast<const float4 *>(srow + 4 * next);
      } else {
        s[p].x = srow[std::min(4 * next + 0, G - 1)];
        s[p].y = srow[std::min(4 * next + 1, G - 1)];
        s[p].z = srow[std::min(4 * next + 2, G - 1)];
        s[p].w = srow[std::min(4 * next + 3, G - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// one chunk of MC (<= MR) slots: row maxima, then per window of W groups the
// limb split and the stream.  Rows past MC of the tile read the zero chunk.
template <int MR, int MC, bool kSc4, bool kOnePass>
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
  const int zchunk = G4 * 4 * MR * 16;
  const float4 *X4 = reinterpret_cast<const float4 *>(X);
  const long K4 = long(K8) * 2;
  const int R_ = lane >> 4;
  constexpr int PD = kMfmaDepth<kSc4>;

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
  for (int p = 0; p < PD; ++p) mfma_load<kSc4>(wrow, srow, G, std::min(p, S - 1), R_, w[p], s[p]);

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

  const int rr = lane & 15;
  const int a_off = rr < MC ? (R_ * MR + rr) * 16 : zchunk;
  const int a_g = rr < MC ? 4 * MR * 16 : 0;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // the ring's first loads (issued before the staging) are in by now; with
  // nothing in flight on entry, the waits inside the stream's loop stay exact
  // (each step waits for its own loads only) instead of draining every ring
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  mfma_stream<MC, kSc4, PD>(xa, a_off, a_g, reg, zchunk, wrow, srow, G, S, 0,
                            (S + PD - 1) / PD * PD, w, s, acc);
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

template <int MR, bool kSc4, bool kOnePass>
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
  if (t == 0) {
    // the zero chunks (never overwritten; the barrier below orders these
    // stores before any read)
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    *reinterpret_cast<float4 *>(xa + G4 * 4 * MR * 16) = z4;
    *reinterpret_cast<float4 *>(xa + reg + G4 * 4 * MR * 16) = z4;
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
    const long nrow = std::min(n0 + (lane & 15), N - 1);
    const uint4 *wrow = qw + (long(e) * N + nrow) * G;
    const float *srow = sc + (long(e) * N + nrow) * G;
    switch (mc) {
      case 1: mfma_chunk<MR, 1, kSc4, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow); break;
      case 2:
        if constexpr (MR >= 2) mfma_chunk<MR, 2, kSc4, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
        break;
      case 3:
        if constexpr (MR >= 4) mfma_chunk<MR, 3, kSc4, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
        break;
      default:
        if constexpr (MR >= 4) mfma_chunk<MR, 4, kSc4, kOnePass>(X, token_index, xa, red, Y, T, N, G, rbase, n0, wrow, srow);
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
                    const int32_t *offsets, const int32_t *qw, const float *sc, float *Y, int T,
                    int R, int E, int N, int G, hipStream_t stream) {
  const uint4 *q = reinterpret_cast<const uint4 *>(qw);
  const bool one_pass = 4 * ((G + 3) & ~3) <= 2 * kMfmaThreads;
#define W4A16_GROUPED_MFMA(SC4, ONE)                                                             \
  hipLaunchKernelGGL((grouped_mfma<MR, SC4, ONE>), dim3(p.grid), dim3(kMfmaThreads), p.lds,      \
                     stream, X, token_index, offsets, q, sc, Y, T, R, E, N, G)
  if (G % 4 == 0) {
    if (one_pass) W4A16_GROUPED_MFMA(true, true);
    else W4A16_GROUPED_MFMA(true, false);
  } else {
    if (one_pass) W4A16_GROUPED_MFMA(false, true);
    else W4A16_GROUPED_MFMA(false, false);
  }
#undef W4A16_GROUPED_MFMA
  return hipGetLastError();
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
  if (plan_mfma(T, R, E, N, G, cus, mp)) {
    switch (mp.MR) {
      case 1: return run_mfma<1>(mp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
      case 2: return run_mfma<2>(mp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
      default: return run_mfma<4>(mp, X, token_index, offsets, qweight, scales, Y, T, R, E, N, G, stream);
    }
  }
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

}  // namespace w4a16
