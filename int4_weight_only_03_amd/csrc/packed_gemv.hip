// Decode GEMV (M <= 4 rows of X) on weights packed by w4a16_grouped_pack
// (one expert): the contraction of the grouped matrix-core kernel, with the
// input dimension split over the waves of a workgroup instead of the columns.
//
// The pages' decode configurations are single-token GEMVs over the MoE and
// MLP weights ("The Quiet Commit: How a Single Plan Update Closed Phase 3 of
// a Native DDTree Inference Engine", section "Input and Output Knowledge":
// the path exists for memory-bound MoE inference and should approach the HBM
// bandwidth peak).  The arithmetic is the split path's (exact weight codes
// q - 8 in fp16, two fp16 limbs of each activation prescaled by a power of
// two, fp32 accumulation, one fp32 FMA per group for the scale), the result
// within the tolerance of w4a16_gemm.
//
// One workgroup of NW waves per 16-row tile of W (8 waves when the tiles fit
// the compute units in one round, else 4):
//  * every thread first reads the activation blocks it will split (or, for
//    long K, reads the rows again later), then every wave issues the loads of
//    its steps (a step: 4 groups of the tile, one contiguous kilobyte of
//    codes in MFMA operand order plus 256 bytes of scales); the global loads
//    complete in issue order, so the activations are not held up behind the
//    weights;
//  * the workgroup stages the M activation rows: each row's maximum gives its
//    exponent, and the limbs go to LDS as MFMA A fragments (16-byte chunk
//    j*M + r holds the 8 limbs of 8-wide block j of row r; a zero region of 4
//    groups follows each limb region); the barriers wait for LDS only, so the
//    weights stay in flight;
//  * wave w contracts steps [w S / NW, (w + 1) S / NW): per group a hi and a
//    lo MFMA into one zeroed 16 x 16 tile (rows 0..M-1 are the activation
//    rows; the others repeat them and are never stored), then one FMA per row
//    with the group's scale;
//  * the waves' partial sums meet in LDS and are added in wave order
//    (deterministic), the row's power of two is undone, Y is written.

#include "w4a16_internal.h"
#include "gemv_common.h"
#include "limbs.h"

#include <algorithm>

namespace w4a16 {
namespace {

constexpr int kPgMaxWaves = 8;
constexpr int kPgSteps = 8;  // steps a wave holds in registers per pass
constexpr int kPgXRegs = 4;  // 8-wide activation blocks a thread may hold (rows x blocks)

__device__ __forceinline__ float pg_absmax(float4 a, float4 c) {
  return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
               fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
}

// LDS writes of this wave complete, then the workgroup barrier; the wave's
// global loads stay in flight
__device__ __forceinline__ void pg_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS bytes: two limb regions of (G4 + 4) groups x 4 blocks x MC chunks, and
// the partial sums [waves][MC][16]
__host__ __device__ constexpr int pg_region_bytes(int MC, int G4) { return (G4 + 4) * 4 * MC * 16; }
__host__ __device__ constexpr int pg_lds_bytes(int MC, int G4) {
  return 2 * pg_region_bytes(MC, G4) + kPgMaxWaves * MC * 16 * 4;
}

// NW waves per workgroup.  kXB > 0: every thread holds its kXB activation
// blocks per row in registers, read before the weights (so that their use
// does not wait for the weights' loads, which complete in order after them);
// kXB == 0: the rows are read twice after the weights (longer K).
template <int MC, int NW, int kXB>
__global__ void __launch_bounds__(64 * NW)
packed_gemv(const float *__restrict__ X, const uint4 *__restrict__ pw, const float *__restrict__ ps,
            float *__restrict__ Y, int N, int G) {
  extern __shared__ __align__(16) unsigned char xa[];
  constexpr int NT = 64 * NW;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int R = lane >> 4;
  const int tile = blockIdx.x;
  const int S = (G + 3) / 4;
  const int G4 = 4 * S;
  const int K8 = 4 * G;
  const int reg = pg_region_bytes(MC, G4);
  const int zregion = G4 * 4 * MC * 16;
  float *red = reinterpret_cast<float *>(xa + 2 * reg);
  constexpr int AG = 4 * MC * 16;  // bytes between consecutive groups' A fragments
  const float4 *X4 = reinterpret_cast<const float4 *>(X);

  // the activation blocks this thread splits, first (kXB > 0)
  float4 xa4[MC][kXB > 0 ? kXB : 1], xc4[MC][kXB > 0 ? kXB : 1];
  if constexpr (kXB > 0) {
#pragma unroll
    for (int r = 0; r < MC; ++r)
#pragma unroll
      for (int u = 0; u < kXB; ++u) {
        const long j = std::min(t + u * NT, K8 - 1);
        xa4[r][u] = X4[long(r) * 2 * K8 + 2 * j];
        xc4[r][u] = X4[long(r) * 2 * K8 + 2 * j + 1];
      }
  }

  // this wave's steps and their loads (clamped into the range; a wave with
  // no step loads step 0 and adds nothing)
  const int s_lo = wave * S / NW, s_hi = (wave + 1) * S / NW;
  const uint4 *wt = pw + long(tile) * S * 64 + lane;
  const float *st = ps + (long(tile) * S * 16 + (lane & 15)) * 4;
  uint4 w[kPgSteps];
  float4 sc[kPgSteps];
#pragma unroll
  for (int p = 0; p < kPgSteps; ++p) {
    const int step = std::max(0, std::min(s_lo + p, s_hi - 1));
    w[p] = load_stream16(wt + long(step) * 64);
    sc[p] = *reinterpret_cast<const float4 *>(st + long(step) * 64);
  }

  // row maxima, exponents
  float mx[MC];
#pragma unroll
  for (int r = 0; r < MC; ++r) mx[r] = 0.0f;
  if constexpr (kXB > 0) {
#pragma unroll
    for (int r = 0; r < MC; ++r)
#pragma unroll
      for (int u = 0; u < kXB; ++u) mx[r] = fmaxf(mx[r], pg_absmax(xa4[r][u], xc4[r][u]));
  } else {
    for (int j = t; j < K8; j += NT) {
#pragma unroll
      for (int r = 0; r < MC; ++r)
        mx[r] = fmaxf(mx[r], pg_absmax(X4[long(r) * 2 * K8 + 2 * j],
                                       X4[long(r) * 2 * K8 + 2 * j + 1]));
    }
  }
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    float v = mx[r];
    for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
    if (lane == 0) red[wave * MC * 16 + r] = v;
  }
  pg_lds_barrier();
  int ex[MC];
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < NW; ++q) v = fmaxf(v, red[q * MC * 16 + r]);
    ex[r] = row_exponent(v);
  }
  // limbs of blocks [0, 4 G4), zero past K, and the zero regions
  if constexpr (kXB > 0) {
#pragma unroll
    for (int u = 0; u < kXB; ++u) {
      const int j = t + u * NT;
      if (j < K8) {
#pragma unroll
        for (int r = 0; r < MC; ++r) {
          half8_t h, l;
          split_block(xa4[r][u], xc4[r][u], ex[r], h, l);
          *reinterpret_cast<half8_t *>(xa + (j * MC + r) * 16) = h;
          *reinterpret_cast<half8_t *>(xa + reg + (j * MC + r) * 16) = l;
        }
      }
    }
    for (int j = K8 + t; j < 4 * G4 + 16; j += NT) {
      const half8_t z = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < MC; ++r) {
        *reinterpret_cast<half8_t *>(xa + (j * MC + r) * 16) = z;
        *reinterpret_cast<half8_t *>(xa + reg + (j * MC + r) * 16) = z;
      }
    }
  } else {
    for (int j = t; j < 4 * G4 + 16; j += NT) {
#pragma unroll
      for (int r = 0; r < MC; ++r) {
        half8_t h, l;
        if (j < K8) {
          split_block(X4[long(r) * 2 * K8 + 2 * j], X4[long(r) * 2 * K8 + 2 * j + 1], ex[r], h, l);
        } else {
          h = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
          l = h;
        }
        *reinterpret_cast<half8_t *>(xa + (j * MC + r) * 16) = h;
        *reinterpret_cast<half8_t *>(xa + reg + (j * MC + r) * 16) = l;
      }
    }
  }
  pg_lds_barrier();  // limbs in; the maxima in red are no longer read

  // the wave's steps, kPgSteps per pass
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int a_off = (R * MC + std::min(lane & 15, MC - 1)) * 16;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = s_lo; s0 < s_hi; s0 += kPgSteps) {
    if (s0 > s_lo) {  // a further pass (more than kPgSteps steps per wave)
#pragma unroll
      for (int p = 0; p < kPgSteps; ++p) {
        const int step = std::min(s0 + p, s_hi - 1);
        w[p] = load_stream16(wt + long(step) * 64);
        sc[p] = *reinterpret_cast<const float4 *>(st + long(step) * 64);
      }
    }
#pragma unroll
    for (int p = 0; p < kPgSteps; ++p) {
      const int step = s0 + p;
      // a step past the wave's range reads the zero region and adds 0
      const unsigned char *ap = xa + (step < s_hi ? a_off + 4 * step * AG : zregion);
      half8_t ah[4], al[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ah[q] = *reinterpret_cast<const half8_t *>(ap + q * AG);
        al[q] = *reinterpret_cast<const half8_t *>(ap + q * AG + reg);
      }
      const half8_t b0 = nibbles_to_f16(w[p].x), b1 = nibbles_to_f16(w[p].y);
      const half8_t b2 = nibbles_to_f16(w[p].z), b3 = nibbles_to_f16(w[p].w);
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
        acc[i] = fmaf(sc[p].x, d0[i], acc[i]);
        acc[i] = fmaf(sc[p].y, d1[i], acc[i]);
        acc[i] = fmaf(sc[p].z, d2[i], acc[i]);
        acc[i] = fmaf(sc[p].w, d3[i], acc[i]);
      }
    }
  }

  // partial sums of the 16 columns (lanes 0..15, rows 0..MC-1), added in
  // wave order
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < MC; ++i) red[(wave * MC + i) * 16 + lane] = acc[i];
  }
  __syncthreads();
  if (t < MC * 16) {
    const int i = t >> 4, c = t & 15;
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < NW; ++q) v += red[(q * MC + i) * 16 + c];
    const int n = tile * 16 + c;
    if (n < N) Y[long(i) * N + n] = ldexpf(v, -ex[i]);
  }
}

template <int MC, int NW>
hipError_t run_pg(const float *X, const uint4 *pw, const float *ps, float *Y, int N, int G,
                  long tiles, size_t lds, hipStream_t stream) {
  constexpr int NT = 64 * NW;
  const int K8 = 4 * G;
  const int xb = (K8 + NT - 1) / NT;  // activation blocks per thread and row
  if (MC * xb <= kPgXRegs) {
    switch (xb) {
      case 1: hipLaunchKernelGGL((packed_gemv<MC, NW, 1>), dim3(unsigned(tiles)), dim3(NT), lds, stream, X, pw, ps, Y, N, G); break;
      case 2: if constexpr (MC <= 2) hipLaunchKernelGGL((packed_gemv<MC, NW, 2>), dim3(unsigned(tiles)), dim3(NT), lds, stream, X, pw, ps, Y, N, G); break;
      default: if constexpr (MC == 1) hipLaunchKernelGGL((packed_gemv<MC, NW, 4>), dim3(unsigned(tiles)), dim3(NT), lds, stream, X, pw, ps, Y, N, G); break;
    }
  } else {
    hipLaunchKernelGGL((packed_gemv<MC, NW, 0>), dim3(unsigned(tiles)), dim3(NT), lds, stream, X, pw, ps, Y, N, G);
  }
  return hipGetLastError();
}

template <int MC>
hipError_t run_pg_waves(const float *X, const uint4 *pw, const float *ps, float *Y, int N, int G,
                        long tiles, size_t lds, int cus, hipStream_t stream) {
  // 8 waves when the tiles fit the compute units in one round; 4 (several
  // workgroups per compute unit) when there are more tiles
  if (tiles <= cus) return run_pg<MC, 8>(X, pw, ps, Y, N, G, tiles, lds, stream);
  return run_pg<MC, 4>(X, pw, ps, Y, N, G, tiles, lds, stream);
}

}  // namespace

bool decode_packed_supported(int M, int K) {
  const int G4 = ((K / kGroup) + 3) / 4 * 4;
  return M >= 1 && M <= 4 && pg_lds_bytes(M, G4) <= 150 * 1024;
}

hipError_t launch_decode_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                                hipStream_t stream) {
  const int G = K / kGroup;
  const int G4 = (G + 3) / 4 * 4;
  const long tiles = (N + 15) / 16;
  if (tiles > 0x7fffffffL || !decode_packed_supported(M, K)) return hipErrorInvalidValue;
  const uint4 *pw = static_cast<const uint4 *>(packed);
  const float *ps = reinterpret_cast<const float *>(pw + tiles * (G4 / 4) * 64);
  const size_t lds = size_t(pg_lds_bytes(M, G4));
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  switch (M) {
    case 1: return run_pg_waves<1>(X, pw, ps, Y, N, G, tiles, lds, cus, stream);
    case 2: return run_pg_waves<2>(X, pw, ps, Y, N, G, tiles, lds, cus, stream);
    case 3: return run_pg_waves<3>(X, pw, ps, Y, N, G, tiles, lds, cus, stream);
    default: return run_pg_waves<4>(X, pw, ps, Y, N, G, tiles, lds, cus, stream);
  }
}

}  // namespace w4a16
