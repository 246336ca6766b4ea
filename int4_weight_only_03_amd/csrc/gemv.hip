// Decode/verify path of the W4A16 GEMM: Y[M][N] = X[M][K] . dequant(W)^T for
// small M, dequantizing on the fly.
//
// The pages build this path for memory-bound MoE inference and name reaching
// the HBM bandwidth peak as its goal ("The Quiet Commit: How a Single Plan
// Update Closed Phase 3 of a Native DDTree Inference Engine", sections "Input
// and Output Knowledge" and "The Thinking Process").  They warn that nibble
// unpacking can eat the bandwidth saved by 4-bit storage ("The Silence of
// Success: A Single Line That Speaks Volumes", section "Assumptions Embedded
// in the Code"), so the inner loop is counted in VALU operations per weight.
//
// Arithmetic (both kernels below):
//  * One 16-byte load brings exactly one group of one W row: 4 words = 32
//    nibbles.  A compute thread owns one group column g and keeps its 32
//    activations in VGPRs for every W row it visits.
//  * Nibbles become signed bytes 16*(q-8) with one or two bit operations per
//    word (mask the high nibbles, or shift-and-mask the low nibbles, then flip
//    bit 7: v_bitop3); each byte converts to fp32 exactly (v_cvt_f32_i32 with a
//    sign-extended SDWA byte select) and meets x in one FMA; the group sum is
//    two fp32 chains (even and odd k), multiplied by 1/16 exactly, and the
//    group's scale multiplies that sum (scale after the 32-term sum).
//  * No atomics: every output is summed in a fixed order, so results are
//    deterministic run to run.
//
// Fast kernel (M <= 2): wave-specialised.  The first kLoaders threads of a
// block stage the activation rows in LDS while every other wave issues all
// of its weight and scale loads straight away (straight-line code, clamped
// row indices, no branches between loads), so the weights stream from the
// first cycle and no wave's in-order load counter ties activations to
// weights.  Partial sums are reduced with DPP row shifts and row broadcasts
// inside aligned lane segments (no LDS round trip), and one LDS pass adds the
// few segment sums of a row.  Blocks are sized so that the grid is about one
// block per compute unit.

#include "w4a16_internal.h"
#include "gemv_common.h"

#include <algorithm>

namespace w4a16 {
namespace {

constexpr int kFastMaxBlock = 768;  // 12 waves: up to 170 VGPRs per lane
constexpr int kLoaders = 128;       // activation-staging threads per block (fast kernel)
constexpr int kXChunk = 16;         // float4 each staging thread moves (32 KB per block)
constexpr int kFastMaxLds = 64 * 1024;


// Fast kernel (M = MT).  Thread t < kLoaders stages the MT rows of X in LDS;
// thread kLoaders + s*G + c (c < G, s < S) is compute thread (slot s, group
// c) for rows rowbase + s + i*S, i < RB.  Z (16, 32 or 64) divides G, so
// segments of Z compute lanes never straddle a slot.
template <int MT, int RB, int Z>
__global__ void __launch_bounds__(kFastMaxBlock)
gemv_ws(const float *__restrict__ X, const uint4 *__restrict__ qw, const float *__restrict__ sc,
        float *__restrict__ Y, int M, int N, int G, int S) {
  extern __shared__ __align__(16) float lds[];
  const long K = long(G) * kGroup;
  const int rowx4 = G * 8;            // float4 per activation row
  const int nx4 = MT * rowx4;         // float4 staged (all M = MT rows)
  float *xs = lds;                    // [MT][K] activations, then one pad float4
  float *part = lds + 4 * (nx4 + 1);  // [segments][MT*RB] segment partial sums
  const int t = threadIdx.x;
  const bool loader = t < kLoaders;
  const int c = t - kLoaders;
  const int slot0 = loader ? 0 : c / G;
  const bool active = !loader && slot0 < S;
  const int slot = active ? slot0 : 0;
  const int g = active ? c - slot0 * G : 0;
  const long rowbase = long(blockIdx.x) * S * RB;
  float acc[MT][RB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[m][i] = 0.0f;
  uint4 w[RB];
  float s[RB];
  if (loader) {  // one straight-line pass: nx4 <= kLoaders * kXChunk
    float4 v[kXChunk];
#pragma unroll
    for (int u = 0; u < kXChunk; ++u) {
      const int k = std::min(t + u * kLoaders, nx4 - 1);
      const int mr = (MT > 1 && k >= rowx4) ? 1 : 0;
      v[u] = reinterpret_cast<const float4 *>(X + mr * K)[k - mr * rowx4];
    }
    // every staging load is issued before the first store waits on one: the
    // empty asm consumes all loaded values at once
#pragma unroll
    for (int u = 0; u < kXChunk; ++u) asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
#pragma unroll
    for (int u = 0; u < kXChunk; ++u)  // out-of-range threads write the pad slot
      reinterpret_cast<float4 *>(xs)[std::min(t + u * kLoaders, nx4)] = v[u];
  } else {
#pragma unroll
    for (int i = 0; i < RB; ++i) {  // clamped rows: no branch between loads
      const long n = std::min(rowbase + slot + long(i) * S, long(N) - 1);
      w[i] = load_stream16(qw + n * G + g);
      s[i] = load_stream4(sc + n * G + g);
    }
  }
  __syncthreads();
  if (!loader) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float x[32];
      const float4 *xp = reinterpret_cast<const float4 *>(xs + m * K + long(g) * kGroup);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 f = xp[v];
        x[4 * v + 0] = f.x;
        x[4 * v + 1] = f.y;
        x[4 * v + 2] = f.z;
        x[4 * v + 3] = f.w;
      }
      // scale * (group sum / 16): the power-of-two 1/16 is exact
#pragma unroll
      for (int i = 0; i < RB; ++i)
        acc[m][i] = active ? s[i] * (group_dot16(x, w[i]) * 0.0625f) : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[m][i] = segment_sum<Z>(acc[m][i]);
    if ((c & (Z - 1)) == Z - 1) {
      const int seg = c / Z;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < RB; ++i) part[seg * (MT * RB) + m * RB + i] = acc[m][i];
    }
  }
  __syncthreads();
  const int sps = G / Z;  // segments per slot
  for (int o = t; o < S * MT * RB; o += blockDim.x) {
    const int sl = o / (MT * RB);
    const int r = o - sl * (MT * RB);
    const int m = r / RB;
    const int i = r - m * RB;
    float v = 0.0f;
    for (int k = 0; k < sps; ++k) v += part[(sl * sps + k) * (MT * RB) + m * RB + i];
    const long n = rowbase + sl + long(i) * S;
    if (m < M && n < N) Y[long(m) * N + n] = v;
  }
}

struct FastPlan {
  int MT, RB, S, Z, BS, blocks;
  size_t lds;
};

// Fast kernel plan: about one block per compute unit (256 on MI355X).
bool plan_fast(int M, int N, int G, FastPlan &p) {
  if (M > 2) return false;
  p.MT = M;  // the fast kernel stages all M rows at once
  p.Z = 1;
  while (p.Z < 64 && G % (2 * p.Z) == 0) p.Z *= 2;
  if (p.Z < 16) return false;  // segments of 16, 32 or 64 lanes only
  const int s_max = (kFastMaxBlock - kLoaders) / G;
  if (s_max < 1) return false;
  const long rows_per_block = std::max(1L, (long(N) + 255) / 256);
  const int prefs[4] = {4, 8, 2, 1};
  p.RB = 0;
  for (int rb : prefs) {
    if (rb * p.MT > 8) continue;  // MT*RB <= 8 partial sums keeps the kernel spill-free
    const long s = (rows_per_block + rb - 1) / rb;
    if (s <= s_max) {
      p.RB = rb;
      p.S = int(s);
      break;
    }
  }
  if (p.RB == 0) {  // very tall W: widest blocks, more of them
    p.RB = 8 / p.MT;
    p.S = s_max;
  }
  if (long(p.MT) * G * 8 > long(kLoaders) * kXChunk) return false;  // one staging pass
  p.BS = ((kLoaders + p.S * G + 63) / 64) * 64;
  p.blocks = int((long(N) + long(p.S) * p.RB - 1) / (long(p.S) * p.RB));
  const size_t segs = size_t(p.BS - kLoaders) / p.Z + 1;
  p.lds = 16 * (size_t(p.MT) * G * 8 + 1) + segs * p.MT * p.RB * sizeof(float);
  return p.lds <= size_t(kFastMaxLds);
}

template <int MT, int RB, int Z>
hipError_t run_fast(const FastPlan &p, const float *X, const int32_t *qw, const float *sc,
                    float *Y, int M, int N, int G, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_ws<MT, RB, Z>), dim3(p.blocks), dim3(p.BS), p.lds, stream, X,
                     reinterpret_cast<const uint4 *>(qw), sc, Y, M, N, G, p.S);
  return hipGetLastError();
}

template <int Z>
hipError_t dispatch_fast_z(const FastPlan &p, const float *X, const int32_t *qw, const float *sc,
                           float *Y, int M, int N, int G, hipStream_t stream) {
  switch (p.MT * 16 + p.RB) {
    case 1 * 16 + 8: return run_fast<1, 8, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 4: return run_fast<1, 4, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 2: return run_fast<1, 2, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 1: return run_fast<1, 1, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 4: return run_fast<2, 4, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 2: return run_fast<2, 2, Z>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 1: return run_fast<2, 1, Z>(p, X, qw, sc, Y, M, N, G, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dispatch_fast(const FastPlan &p, const float *X, const int32_t *qw, const float *sc,
                         float *Y, int M, int N, int G, hipStream_t stream) {
  switch (p.Z) {
    case 64: return dispatch_fast_z<64>(p, X, qw, sc, Y, M, N, G, stream);
    case 32: return dispatch_fast_z<32>(p, X, qw, sc, Y, M, N, G, stream);
    case 16: return dispatch_fast_z<16>(p, X, qw, sc, Y, M, N, G, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// General kernel (any M, any K): each thread loads its activations straight
// from memory.  One block covers S*RB consecutive W rows.  Thread t: slot =
// t / TPS, column c = t % TPS; slot s handles rows rowbase + s + i*S (i < RB)
// and groups c, c+TPS, ... .  T = lanes per reduction team (power of two <= 64).

constexpr int kMaxBlock = 512;  // 8 waves per block leaves up to 256 VGPRs per lane

template <int MT, int RB>
__global__ void __launch_bounds__(kMaxBlock)
gemv_w4a16(const float *__restrict__ X, const uint4 *__restrict__ qw,
           const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G, int S,
           int TPS, int T) {
  extern __shared__ float red[];  // [MT*RB][blockDim.x + 1]
  const int BS = blockDim.x;
  const int ld = BS + 1;
  const int t = threadIdx.x;
  const int slot = t / TPS;
  const int col = t - slot * TPS;
  const bool active = slot < S;
  const long rowbase = long(blockIdx.x) * S * RB;
  const long K = long(G) * kGroup;

  for (int m0 = 0; m0 < M; m0 += MT) {
    float acc[MT][RB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[m][i] = 0.0f;

    if (active) {
      for (int g = col; g < G; g += TPS) {
        uint4 w[RB];
        float s[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {  // clamped rows: no branch between loads
          const long n = std::min(rowbase + slot + long(i) * S, long(N) - 1);
          w[i] = load_stream16(qw + n * G + g);
          s[i] = load_stream4(sc + n * G + g);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float x[32];
          const int row = std::min(m0 + m, M - 1);  // rows past M are computed and dropped
          const float4 *xp = reinterpret_cast<const float4 *>(X + long(row) * K + long(g) * kGroup);
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

    const int O = MT * S * RB;  // outputs of this block and m-tile
    const int team = t / T;
    const int j = t - team * T;
    const int teams = BS / T;
    for (int o = team; o < O; o += teams) {
      const int m = o / (S * RB);
      const int r = o - m * S * RB;
      const int i = r / S;
      const int sl = r - i * S;
      const float *src = red + (m * RB + i) * ld + sl * TPS;
      float v = 0.0f;
      for (int c = j; c < TPS; c += T) v += src[c];
      for (int d = T >> 1; d > 0; d >>= 1) v += __shfl_xor(v, d, T);
      const long n = rowbase + sl + long(i) * S;
      if (j == 0 && m0 + m < M && n < N) Y[long(m0 + m) * N + n] = v;
    }
    __syncthreads();
  }
}

struct GemvPlan {
  int TPS, S, BS, RB, MT, T, blocks;
};

int pow2_floor(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}

// 256 CUs x ~7 resident waves: enough 16-byte loads in flight to cover HBM latency.
constexpr long kTargetThreads = 256L * 7 * 64;

GemvPlan plan_gemv(int M, int N, int G) {
  GemvPlan p;
  p.TPS = std::min(G, kMaxBlock);
  p.MT = M >= 3 ? 4 : (M == 2 ? 2 : 1);
  // Rows per thread: as many as keep ~kTargetThreads threads busy (amortizes
  // the activation loads), at least 1.
  const long chunks = long(N) * p.TPS;
  p.RB = 8 / p.MT;  // MT*RB <= 8 partial sums per thread keeps VGPRs below 256
  while (p.RB > 1 && chunks / p.RB < kTargetThreads) p.RB /= 2;
  // Slots per block: the count with the fewest idle lanes in whole waves,
  // the smaller count on ties.
  int best_s = 1, best_idle = 1 << 30;
  for (int s = 1; s * p.TPS <= kMaxBlock; ++s) {
    const int bs = ((s * p.TPS + 63) / 64) * 64;
    const int idle_per_1024 = (bs - s * p.TPS) * 1024 / bs;
    if (idle_per_1024 < best_idle) {
      best_idle = idle_per_1024;
      best_s = s;
    }
  }
  p.S = best_s;
  p.BS = ((p.S * p.TPS + 63) / 64) * 64;
  p.blocks = int((long(N) + long(p.S) * p.RB - 1) / (long(p.S) * p.RB));
  const int O = p.MT * p.S * p.RB;
  p.T = std::min(64, std::max(1, pow2_floor(std::max(1, p.BS / O))));
  return p;
}

template <int MT, int RB>
hipError_t run(const GemvPlan &p, const float *X, const int32_t *qw, const float *sc, float *Y,
               int M, int N, int G, hipStream_t stream) {
  if (p.MT != MT || p.RB != RB) return hipErrorInvalidValue;  // plan and kernel must agree
  const size_t lds = size_t(MT) * RB * (p.BS + 1) * sizeof(float);
  hipLaunchKernelGGL((gemv_w4a16<MT, RB>), dim3(p.blocks), dim3(p.BS), lds, stream, X,
                     reinterpret_cast<const uint4 *>(qw), sc, Y, M, N, G, p.S, p.TPS, p.T);
  return hipGetLastError();
}

hipError_t dispatch(const GemvPlan &p, const float *X, const int32_t *qw, const float *sc,
                    float *Y, int M, int N, int G, hipStream_t stream) {
  switch (p.MT * 16 + p.RB) {
    case 1 * 16 + 8: return run<1, 8>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 4: return run<1, 4>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 2: return run<1, 2>(p, X, qw, sc, Y, M, N, G, stream);
    case 1 * 16 + 1: return run<1, 1>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 4: return run<2, 4>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 2: return run<2, 2>(p, X, qw, sc, Y, M, N, G, stream);
    case 2 * 16 + 1: return run<2, 1>(p, X, qw, sc, Y, M, N, G, stream);
    case 4 * 16 + 2: return run<4, 2>(p, X, qw, sc, Y, M, N, G, stream);
    case 4 * 16 + 1: return run<4, 1>(p, X, qw, sc, Y, M, N, G, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch(const float *X, const int32_t *qweight, const float *scales, float *Y, int M,
                  int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  FastPlan fp;
  if (plan_fast(M, N, G, fp)) return dispatch_fast(fp, X, qweight, scales, Y, M, N, G, stream);
  return dispatch(plan_gemv(M, N, G), X, qweight, scales, Y, M, N, G, stream);
}

}  // namespace

// From 5 rows the decode GEMV carries four A operands per weight word (8
// rows' limbs), and on a weight matrix of at least 4096 x 4096 the skinny
// kernel, which then fills the chip with 16-row tiles, is the faster one
// (measured on MI355X: 13.0 against 17.4 us at 8 x 4096 x 7168, 20.1 against
// 24.9 at 8 x 14336 x 4096; below that size the two are even or the GEMV
// wins, 9.5 against 11.7 us at 8 x 1024 x 7168).
bool skinny_beats_decode_gemv(int M, int N, int K) { return M >= 5 && N >= 4096 && K >= 4096; }

int gemv_kernel(int M, int N, int K) {
  if (gemv_mfma_supported(M, K) && !skinny_beats_decode_gemv(M, N, K))
    return W4A16_GEMV_MFMA;  // matrix-core decode GEMV
  if (M >= 3 && skinny_supported(M)) return W4A16_GEMV_SKINNY;  // skinny.hip
  return W4A16_GEMV_FMA;
}

hipError_t launch_gemv(const float *X, const int32_t *qweight, const float *scales, float *Y,
                       int M, int N, int K, hipStream_t stream) {
  switch (gemv_kernel(M, N, K)) {
    case W4A16_GEMV_MFMA: return launch_gemv_mfma(X, qweight, scales, Y, M, N, K, stream);
    case W4A16_GEMV_SKINNY: return launch_skinny(X, qweight, scales, Y, M, N, K, stream);
    default: return launch(X, qweight, scales, Y, M, N, K, stream);
  }
}

hipError_t launch_gemv_fma(const float *X, const int32_t *qweight, const float *scales, float *Y,
                           int M, int N, int K, hipStream_t stream) {
  return launch(X, qweight, scales, Y, M, N, K, stream);
}

hipError_t launch_gemv_swiglu(const float *X, const int32_t *qweight, const float *scales,
                              float *Y, int M, int F, int K, hipStream_t stream) {
  // the same choice as launch_gemv over the 2F rows of W (measured: 15.0
  // against 18.8 us at 8 x 2*2048 x 7168 on the skinny kernel's fused form)
  if (gemv_kernel(M, 2 * F, K) == W4A16_GEMV_MFMA)  // matrix-core decode GEMV (gemv_mfma.hip)
    return launch_gemv_mfma_swiglu(X, qweight, scales, Y, M, F, K, stream);
  return launch_skinny_swiglu(X, qweight, scales, Y, M, F, K, stream);  // skinny.hip
}

}  // namespace w4a16
