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
//    (4 x J MFMA tiles of 16 x 16).  Work moves in quads of 4 groups: the
//    activation limbs of a quad are copied straight from global memory into an
//    XOR-swizzled LDS image (double-buffered); each lane loads one 16-byte
//    chunk (a whole group) per n-subtile, and a 4 x 4 transpose across lane
//    quarters (v_permlane32_swap, v_permlane16_swap) gives lane quarter kb
//    word kb of each of the 4 groups, the layout the MFMA's B operand wants.
//    Nibbles become f16 (q - 8) pairs with a mask-or into the mantissa of 1024
//    (v_bitop3) and one packed subtract (or a packed FMA for the nibbles that
//    sit 4 bits up).  The MFMAs of one (group, m-subtile) unit run while the
//    previous unit's results are scaled into the accumulators.
//  * The K range may be split over gridDim.y workgroups; each writes its
//    partial tile to the workspace and split_reduce adds the partials in split
//    order (deterministic), undoes the row's power of two and stores Y.

#include "w4a16_internal.h"

#include <algorithm>
#include <cmath>

namespace w4a16 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 64;      // rows of X / Y per workgroup tile
constexpr int kWaves = 4;    // waves per workgroup, side by side along n
constexpr int kQuadK = 128;  // k per quad (4 groups)

// ---------------------------------------------------------------- prep

constexpr int kPrepThreads = 256;
constexpr int kPrepRegBlocks = 4;  // 8-wide k blocks a thread keeps in registers

__device__ __forceinline__ float block_max(float v, float *red) {
  for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// exponent e with max|x| * 2^e in [2^14, 2^15); 0 for a zero or non-finite max
__device__ __forceinline__ int row_exponent(float mx) {
  int e = 0;
  if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
    int E;
    frexpf(mx, &E);  // mx in [2^(E-1), 2^E)
    e = 15 - E;
  }
  return e;
}

__device__ __forceinline__ void split_block(const float4 a, const float4 c, int e, half8_t &h,
                                            half8_t &l) {
  const float v[8] = {a.x, c.x, a.y, c.y, a.z, c.z, a.w, c.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xs = ldexpf(v[i], e);
    const _Float16 hv = (_Float16)xs;
    h[i] = hv;
    l[i] = (_Float16)(xs - (float)hv);
  }
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

// f16 (q - 8) pairs from one word of 8 nibbles: VGPR p holds nibbles p, p+4.
// (w & mask) | 0x6400 puts a nibble into the mantissa of 1024 (v_bitop3).
__device__ __forceinline__ half8_t nibbles_to_f16(uint32_t w) {
  const uint32_t t = w >> 8;
  const half2_t p0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64006400u, 0xEA));
  const half2_t p1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64006400u, 0xEA));
  const half2_t p2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(t, 0x000F000Fu, 0x64006400u, 0xEA));
  const half2_t p3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(t, 0x00F000F0u, 0x64006400u, 0xEA));
  const half2_t c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const half2_t c16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t r0 = p0 - c1032;       // (1024 + q) - 1032
  const half2_t r1 = p1 * c16 - c72;   // (1024 + 16q) / 16 - 72
  const half2_t r2 = p2 - c1032;
  const half2_t r3 = p3 * c16 - c72;
  half8_t o;
  o[0] = r0[0]; o[1] = r0[1]; o[2] = r1[0]; o[3] = r1[1];
  o[4] = r2[0]; o[5] = r2[1]; o[6] = r3[0]; o[7] = r3[1];
  return o;
}

// 4 x 4 transpose across lane quarters: on entry register j of quarter q holds
// word j of quarter q's group; on exit register j of quarter q holds word q of
// group j.
__device__ __forceinline__ void quarter_transpose(uint32_t &r0, uint32_t &r1, uint32_t &r2,
                                                  uint32_t &r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  r0 = a[0];
  r2 = a[1];
  r1 = b[0];
  r3 = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
  auto d = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

__device__ __forceinline__ uint4 load_stream16(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// LDS image of one quad of activation limbs: 2 limbs x 64 rows x 16 chunks of
// 16 bytes (8 f16 of k each).  Chunk c of row r sits at slot c ^ (r & 15) of
// the row, so that the 16 rows one MFMA operand read touches fall in 16
// different bank groups (ds_read_b128 without conflicts, no padding).  The
// image is filled straight from global memory (global_load_lds_dwordx4): slot
// u * 256 + t of the image is loaded by thread t, instruction u, so that each
// wave instruction writes 1 KB of consecutive slots.
constexpr int kImgBytes = 2 * kBM * 16 * 16;  // 32 KB

// Grid: x = output tile, y = K split.  Tiles are numbered m-tile major, n-tile
// minor; when their count divides by 8, workgroup b (the hardware deals
// workgroups round-robin to the 8 XCDs) takes tile (b % 8) * (tiles / 8) + b / 8,
// so that each XCD works through a contiguous run of tiles and its L2 serves
// the rows of X and W those tiles share.
template <int J>
__global__ void __launch_bounds__(kWaves * 64)
split_gemm(const _Float16 *__restrict__ xl, const int *__restrict__ rexp,
           const uint32_t *__restrict__ qw, const float *__restrict__ sc, float *__restrict__ Y,
           float *__restrict__ partial, int M, int N, int G, int n_tiles) {
  constexpr int kBN = kWaves * 16 * J;
  __shared__ __align__(16) unsigned char abuf[2 * kImgBytes];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int l16 = lane & 15;
  const int kb = lane >> 4;
  const long K = long(G) * kGroup;
  const int tiles = gridDim.x;
  int tile = blockIdx.x;
  if ((tiles & 7) == 0) tile = (tile & 7) * (tiles >> 3) + (tile >> 3);
  const int m_tile = tile / n_tiles;
  const int n_tile = tile - m_tile * n_tiles;
  const int split = blockIdx.y;
  const int S = gridDim.y;
  const int m_base = m_tile * kBM;
  const int n_base = n_tile * kBN + wave * 16 * J;
  const int quads = (G + 3) / 4;
  const int q0 = int((long(quads) * split) / S);
  const int q1 = int((long(quads) * (split + 1)) / S);

  // weight rows of this lane, one per n-subtile (rows past N read row N-1)
  const uint4 *wrow[J];
  const float *srow[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int n = std::min(n_base + 16 * j + l16, N - 1);
    wrow[j] = reinterpret_cast<const uint4 *>(qw + long(n) * (long(G) * 4));
    srow[j] = sc + long(n) * G;
  }

  // this thread's chunks of the image: instruction u fills slot u * 256 + t,
  // i.e. limb u / 4, row (u % 4) * 16 + t / 16, chunk column c (the same for
  // every u, since row % 16 = t / 16)
  const int c_col = (t & 15) ^ (t >> 4);
  const _Float16 *arow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = std::min(m_base + v * 16 + (t >> 4), M - 1);
    arow[v] = xl + long(m) * K;
  }
  const long limb_stride = long(M) * K;
  auto issue_a = [&](int q, int img) {
    // a chunk past K reads the row's last chunk instead; its group weighs 0
    const long k = std::min(long(q) * kQuadK + c_col * 8, K - 8);
    unsigned char *dst = abuf + img * kImgBytes + wave * 64 * 16;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_global_load_lds(arow[u & 3] + (u >> 2) * limb_stride + k,
                                       (lds_void *)(dst + u * (kWaves * 64) * 16), 16, 0, 0);
  };
  uint4 wst[J];
  float sst[J][4];
  auto load_w = [&](int q) {
    const int g = std::min(4 * q + kb, G - 1);
#pragma unroll
    for (int j = 0; j < J; ++j) wst[j] = load_stream16(wrow[j] + g);
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int g2 = 4 * q + gg;
        const float v = srow[j][std::min(g2, G - 1)];
        sst[j][gg] = g2 < G ? v : 0.0f;  // groups past G weigh nothing
      }
  };

  floatx4 acc[4][J];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  if (q0 < q1) {
    issue_a(q0, 0);
    load_w(q0);
  }
  for (int q = q0; q < q1; ++q) {
    const int img = (q - q0) & 1;
    // this quad's image is in LDS and every wave is done with the other one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t wr[J][4];
    float s[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      wr[j][0] = wst[j].x;
      wr[j][1] = wst[j].y;
      wr[j][2] = wst[j].z;
      wr[j][3] = wst[j].w;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) s[j][gg] = sst[j][gg];
    }
    if (q + 1 < q1) {
      issue_a(q + 1, img ^ 1);
      load_w(q + 1);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) quarter_transpose(wr[j][0], wr[j][1], wr[j][2], wr[j][3]);
    const unsigned char *ab = abuf + img * kImgBytes;

    // unit (gg, i): 2 J MFMAs into d; the previous unit's d is scaled into acc
    // meanwhile, so that MFMA and VALU work of adjacent units overlap
    floatx4 dp[J];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      half8_t b[J];
#pragma unroll
      for (int j = 0; j < J; ++j) b[j] = nibbles_to_f16(wr[j][gg]);
      const int slot = (gg * 4 + kb) ^ l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + l16;
        const half8_t ahi = *reinterpret_cast<const half8_t *>(ab + (row * 16 + slot) * 16);
        const half8_t alo =
            *reinterpret_cast<const half8_t *>(ab + ((kBM + row) * 16 + slot) * 16);
        floatx4 d[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
          d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b[j], floatx4{0.0f, 0.0f, 0.0f, 0.0f},
                                                        0, 0, 0);
          d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b[j], d[j], 0, 0, 0);
        }
        if (gg + i > 0) {
          const int pi = (i + 3) & 3;
          const int pg = i == 0 ? gg - 1 : gg;
#pragma unroll
          for (int j = 0; j < J; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pi][j][r] = fmaf(dp[j][r], s[j][pg], acc[pi][j][r]);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) dp[j] = d[j];
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[3][j][r] = fmaf(dp[j][r], s[j][3], acc[3][j][r]);
  }

  // lane (l16, kb) of wave w holds rows m_base + 16 i + 4 kb + r of column
  // n_base + 16 j + l16.  One split: Y directly (the row's power of two
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
        const int n = n_base + 16 * j + l16;
        if (n < N) out[long(m) * N + n] = ldexpf(acc[i][j][r], -e);
      }
    }
}

// Y = 2^-e(m) * (sum over splits in order of the partials): one float4 of
// outputs per thread when N % 4 == 0, else one output.
template <bool kVec4>
__global__ void __launch_bounds__(256)
split_reduce(const float *__restrict__ partial, const int *__restrict__ rexp,
             float *__restrict__ Y, int M, int N, int S) {
  const long total = long(M) * N;
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  if constexpr (kVec4) {
    if (4 * i >= total) return;
    float4 v = reinterpret_cast<const float4 *>(partial)[i];
    for (int z = 1; z < S; ++z) {
      const float4 p = reinterpret_cast<const float4 *>(partial + long(z) * total)[i];
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    const int e = rexp[(4 * i) / N];
    reinterpret_cast<float4 *>(Y)[i] =
        make_float4(ldexpf(v.x, -e), ldexpf(v.y, -e), ldexpf(v.z, -e), ldexpf(v.w, -e));
  } else {
    if (i >= total) return;
    float v = partial[i];
    for (int z = 1; z < S; ++z) v += partial[long(z) * total + i];
    Y[i] = ldexpf(v, -rexp[i / N]);
  }
}

struct SplitPlan {
  int J, m_tiles, n_tiles, S;
  size_t off_exp, off_partial, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

SplitPlan make_plan(int M, int N, int G, int J, int S) {
  SplitPlan p;
  p.J = J;
  p.S = S;
  p.m_tiles = (M + kBM - 1) / kBM;
  p.n_tiles = (N + kWaves * 16 * J - 1) / (kWaves * 16 * J);
  const size_t limbs = size_t(2) * M * size_t(G) * kGroup * sizeof(_Float16);
  p.off_exp = 0 + align256(limbs);
  p.off_partial = p.off_exp + align256(size_t(M) * sizeof(int));
  p.bytes = align256(p.off_partial + (S > 1 ? size_t(S) * M * size_t(N) * sizeof(float) : 0));
  return p;
}

// Tile width and K split: the K range is split (powers of two, at least 2
// quads per split) until the grid covers the 256 compute units; among tile
// widths 256, 128 and 64 the one with the smallest estimated time wins, the
// estimate adding per-workgroup MFMA time, its L2 traffic and the split-K
// partials' round trip.
SplitPlan plan_split(int M, int N, int G) {
  const int quads = (G + 3) / 4;
  SplitPlan best{};
  double best_cost = 0.0;
  for (int J : {4, 2, 1}) {
    const int m_tiles = (M + kBM - 1) / kBM;
    const int n_tiles = (N + kWaves * 16 * J - 1) / (kWaves * 16 * J);
    int S = 1;
    while (long(m_tiles) * n_tiles * S < 256 && quads / (S * 2) >= 2) S *= 2;
    const double kq = double(quads) * kQuadK / S;            // k per workgroup
    const double bn = kWaves * 16.0 * J;
    const double mfma_us = kBM * bn * kq * 4.0 / 4.9e6;       // two limbs, ~half of peak
    const double l2_us = (kBM * kq * 4.0 + bn * kq * 0.625) / 1.5e5;
    const double rounds = std::ceil(double(m_tiles) * n_tiles * S / 256.0);
    double cost = rounds * std::max(mfma_us, l2_us);
    if (S > 1) cost += 2.0 * S * double(M) * N * 4.0 / 5e6 + 1.2;
    if (J == 4 || cost < best_cost) {
      best = make_plan(M, N, G, J, S);
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_plan(const SplitPlan &p, const float *X, const int32_t *qweight,
                       const float *scales, float *Y, int M, int N, int K, void *workspace,
                       hipStream_t stream) {
  const int G = K / kGroup;
  char *ws = static_cast<char *>(workspace);
  _Float16 *xl = reinterpret_cast<_Float16 *>(ws);
  int *rexp = reinterpret_cast<int *>(ws + p.off_exp);
  float *partial = reinterpret_cast<float *>(ws + p.off_partial);
  const long tiles = long(p.m_tiles) * p.n_tiles;
  if (tiles > 0x7fffffffL || p.S > 65535) return hipErrorInvalidConfiguration;
  if (K <= 8 * kPrepThreads * kPrepRegBlocks)
    hipLaunchKernelGGL(split_prep<true>, dim3(M), dim3(kPrepThreads), 0, stream, X, xl, rexp, M,
                       K);
  else
    hipLaunchKernelGGL(split_prep<false>, dim3(M), dim3(kPrepThreads), 0, stream, X, xl, rexp, M,
                       K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(unsigned(tiles), unsigned(p.S));
  const auto qw = reinterpret_cast<const uint32_t *>(qweight);
  switch (p.J) {
    case 4:
      hipLaunchKernelGGL(split_gemm<4>, grid, dim3(kWaves * 64), 0, stream, xl, rexp, qw, scales,
                         Y, partial, M, N, G, p.n_tiles);
      break;
    case 2:
      hipLaunchKernelGGL(split_gemm<2>, grid, dim3(kWaves * 64), 0, stream, xl, rexp, qw, scales,
                         Y, partial, M, N, G, p.n_tiles);
      break;
    default:
      hipLaunchKernelGGL(split_gemm<1>, grid, dim3(kWaves * 64), 0, stream, xl, rexp, qw, scales,
                         Y, partial, M, N, G, p.n_tiles);
      break;
  }
  e = hipGetLastError();
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

}  // namespace

size_t split_workspace_bytes(int M, int N, int K) { return plan_split(M, N, K / kGroup).bytes; }

hipError_t launch_split(const float *X, const int32_t *qweight, const float *scales, float *Y,
                        int M, int N, int K, void *workspace, hipStream_t stream) {
  return launch_plan(plan_split(M, N, K / kGroup), X, qweight, scales, Y, M, N, K, workspace,
                     stream);
}

size_t split_workspace_bytes_with(int M, int N, int K, int J, int S) {
  return make_plan(M, N, K / kGroup, J, S).bytes;
}

hipError_t launch_split_with(const float *X, const int32_t *qweight, const float *scales,
                             float *Y, int M, int N, int K, int J, int S, void *workspace,
                             hipStream_t stream) {
  if ((J != 1 && J != 2 && J != 4) || S < 1) return hipErrorInvalidValue;
  return launch_plan(make_plan(M, N, K / kGroup, J, S), X, qweight, scales, Y, M, N, K,
                     workspace, stream);
}

}  // namespace w4a16
