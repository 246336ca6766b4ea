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
// Mapping (gfx950, wave64):
//  * A thread owns one group column g (32 consecutive k) and keeps the 32
//    activations of that group in VGPRs for every W row it visits, so the
//    activation vector is read once per thread, not once per weight.
//  * One 16-byte load (global_load_dwordx4) brings exactly one group of one W
//    row: 4 words = 32 nibbles.  A row slot of TPS = G threads reads one W row
//    as one contiguous run; consecutive slots read consecutive rows, so a wave
//    reads contiguous memory.  Each thread issues all RB row loads (and their
//    scales) before it touches any of them.
//  * Nibbles become signed bytes 16*(q-8) with one or two bit operations per
//    word (mask the high nibbles, or shift-and-mask the low nibbles, then flip
//    bit 7: v_bitop3); each byte converts to fp32 exactly (v_cvt_f32_i32 with a
//    sign-extended SDWA byte select) and meets x in one FMA; the group sum is
//    two fp32 chains (even and odd k), then multiplied by 1/16 exactly.
//  * The group's scale multiplies the 32-term group sum (scale-after-sum);
//    the per-thread partials of a row are summed across the slot in LDS and
//    by a shuffle tree within aligned lane teams.  No atomics: results are
//    deterministic run to run.

#include "w4a16_internal.h"

#include <algorithm>

namespace w4a16 {
namespace {

// Block size cap: 8 waves per block leaves up to 256 VGPRs per lane.
constexpr int kMaxBlock = 512;

// sum over the group of x_k * 16*(q_k - 8): the 16*(q-8) are exact signed
// bytes, each met by one fp32 FMA (one rounding per term).
__device__ __forceinline__ float group_dot16(const float (&x)[32], uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte b of hi: high nibble of byte b (k = 8j+2b+1) in bits 4..7, sign bit flipped
    const uint32_t hi = (u[j] & 0xF0F0F0F0u) ^ 0x80808080u;
    // byte b of lo: low nibble of byte b (k = 8j+2b) moved to bits 4..7, sign bit flipped
    const uint32_t lo = ((u[j] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a0 = fmaf(x[8 * j + 2 * b], float(int8_t(lo >> (8 * b))), a0);
      a1 = fmaf(x[8 * j + 2 * b + 1], float(int8_t(hi >> (8 * b))), a1);
    }
  }
  return a0 + a1;
}

// One block covers S*RB consecutive W rows.  Thread t: slot = t / TPS, column
// c = t % TPS; slot s handles rows rowbase + s + i*S (i < RB) and groups
// c, c+TPS, ... .  T = lanes per reduction team (power of two <= 64).
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
        for (int i = 0; i < RB; ++i) {
          const long n = rowbase + slot + long(i) * S;
          if (n < N) {
            w[i] = qw[n * G + g];
            s[i] = sc[n * G + g];
          } else {
            w[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
            s[i] = 0.0f;
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float x[32];
          if (m0 + m < M) {
            const float4 *xp = reinterpret_cast<const float4 *>(X + long(m0 + m) * K + long(g) * kGroup);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              const float4 f = xp[v];
              x[4 * v + 0] = f.x;
              x[4 * v + 1] = f.y;
              x[4 * v + 2] = f.z;
              x[4 * v + 3] = f.w;
            }
          } else {
#pragma unroll
            for (int v = 0; v < 32; ++v) x[v] = 0.0f;
          }
          // scale * (group sum / 16): the power-of-two 1/16 is exact
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

}  // namespace

hipError_t launch_gemv(const float *X, const int32_t *qweight, const float *scales, float *Y,
                       int M, int N, int K, hipStream_t stream) {
  const int G = K / kGroup;
  return dispatch(plan_gemv(M, N, G), X, qweight, scales, Y, M, N, G, stream);
}

}  // namespace w4a16
