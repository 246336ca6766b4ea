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

#include <algorithm>

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

hipError_t launch_grouped(const float *X, const int32_t *token_index, const int32_t *offsets,
                          const int32_t *qweight, const float *scales, float *Y, int T, int R,
                          int E, int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  if (E > 65535) return hipErrorInvalidConfiguration;
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
