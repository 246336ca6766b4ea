// Large-M W4A16 GEMM on the fp16 matrix cores, with no workspace:
// Y[M][N] = X[M][K] . dequant(W)^T for the compute-bound shapes (the pages'
// prefill-sized products).
//
// Arithmetic: the skinny kernel's (exact weight codes q - 8 in fp16; each fp32
// activation scaled by a power of two per row and pair of groups, the pair's
// largest magnitude into [2^14, 2^15), and split into hi = f16(x 2^e) and
// lo = f16((x 2^e - hi) 2^11), the low limb met by the codes times 2^-11 so
// both limbs' exact products land in one fp32 accumulator; the group scale
// with one fp32 FMA per group into the pair's sum, 2^-e with one FMA per pair
// into the total).  fp32 activations, int4 weights and fp32 accumulation as
// the pages define the operation ("The Silence of Success: A Single Line That
// Speaks Volumes", sections "What the Edit Actually Built" and "Assumptions
// Embedded in the Code").
//
// Mapping: v_mfma_f32_16x16x32_f16, A = limbs of 16 rows of X, B = codes of
// 16 rows of W, K = one group.  Lane (c, R) (c = lane % 16, R = lane / 16)
// holds k = 8R .. 8R+7 of row c of A and of W row c (word R of the group),
// and D[4R + r][c].  A workgroup computes a 128 x 128 tile with 8 waves; wave
// (wm, wn) = (wave / 2, wave % 2) owns rows wm*32 .. +31 of X (2 row tiles u)
// and rows wn*64 .. +63 of W (4 column tiles t).
//
// Pipeline, per pair of groups p (one s_barrier each):
//   * the raw fp32 activations of pair p + 2 are copied into LDS (direct
//     copies, 1 KB per instruction, each row's 16 chunks XOR-swizzled);
//   * the workgroup splits pair p + 1 once (wave w takes rows 16w .. 16w+15:
//     the pair's row maximum over 4 lanes, the exponent, the limbs) and writes
//     the limbs and the factors 2^-e to LDS;
//   * every wave reads pair p's limbs and factors, converts its W rows' codes
//     and runs pair p's matrix instructions.
// The split of pair p + 1 and the products of pair p are independent, so one
// wave's conversions overlap its own matrix instructions.  Raw, limb, weight
// and scale images alternate in pairs of separate __shared__ objects (so the
// compiler can tell the reads of one from the copies into the other).

#include "w4a16_internal.h"
#include "limbs.h"

#include <algorithm>

namespace w4a16 {
namespace {

typedef __attribute__((address_space(3))) void lx_lds_void;

constexpr int kLxWaves = 8;

__device__ __forceinline__ void lx_wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x70 | (15 << 8));  // vmcnt(0)
}
__device__ __forceinline__ void lx_wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | 0x70);  // lgkmcnt(0)
}
// Workgroup barrier without the release fence of __syncthreads() (which would
// wait for the next pairs' copies as well).
__device__ __forceinline__ void lx_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(64 * kLxWaves)
tile_mx(const float *__restrict__ X, const uint32_t *__restrict__ qw,
        const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G, int tiles_n) {
  // raw activations of a pair: row r at 256 r, logical chunk L (k = 4L..4L+3
  // of the pair) at physical chunk L ^ (r % 16)
  __shared__ __align__(16) unsigned char lx_x0[128 * 256];
  __shared__ __align__(16) unsigned char lx_x1[128 * 256];
  // limbs of a pair: row r at 256 r, logical chunk 8 limb + 4 q + b (limb 0 =
  // hi, 1 = lo; group q; k = 8b .. 8b+7 of the group, in the order the nibble
  // conversion produces) at physical chunk (8 limb + 4 q + b) ^ (r % 16)
  __shared__ __align__(16) unsigned char lx_l0[128 * 256];
  __shared__ __align__(16) unsigned char lx_l1[128 * 256];
  // weight words of 4 groups: row n at 64 n, group g at position g ^ ((n / 4) % 4)
  __shared__ __align__(16) unsigned char lx_w0[128 * 64];
  __shared__ __align__(16) unsigned char lx_w1[128 * 64];
  // scales of 4 groups: row n at 16 n
  __shared__ __align__(16) unsigned char lx_s0[128 * 16];
  __shared__ __align__(16) unsigned char lx_s1[128 * 16];
  // 2^-e of a pair, per row
  __shared__ __align__(16) float lx_f0[128];
  __shared__ __align__(16) float lx_f1[128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int c = lane & 15, R = lane >> 4;
  // The hardware deals workgroups round-robin to the 8 XCDs: when the tile
  // count divides by 8, XCD x takes the contiguous run of tiles x*(tiles/8)..
  int tile = blockIdx.x;
  if (gridDim.x % 8 == 0) tile = int(blockIdx.x % 8) * int(gridDim.x / 8) + int(blockIdx.x / 8);
  const int bm = tile / tiles_n;
  const int bn = tile - bm * tiles_n;
  const int m0 = bm * 128, n0 = bn * 128;
  const long K = long(G) * kGroup;
  const int P = (G + 1) / 2;  // pairs of groups (the last may hold one)

  // X copy j (this wave issues j = 4 wave .. 4 wave + 3 of 32): lane i writes
  // 16 B at image offset 1024 j + 16 i: tile row 4j + i/16, physical chunk
  // i % 16, which holds logical chunk (i % 16) ^ (row % 16).  Rows past M read
  // row M-1 (never stored).  Offsets relative to the tile's first row (< 2^26).
  uint32_t xoff[4];
  bool xhigh[4];  // the lane reads the pair's second group
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int row = 4 * (4 * wave + jj) + lane / 16;
    const int L = (lane & 15) ^ (row & 15);
    xhigh[jj] = L >= 8;
    xoff[jj] = uint32_t(std::min(m0 + row, M - 1) - m0) * uint32_t(K * 4) + 16u * uint32_t(L);
  }
  const char *xtile = reinterpret_cast<const char *>(X) + long(m0) * K * 4;
  // W copy (this wave issues copy `wave` of 8): lane i writes 16 B at offset
  // 1024 wave + 16 i: tile row 16 wave + i/4, position i % 4, which holds group
  // (i % 4) ^ ((row / 4) % 4) of the 4-group block.  Scale copy: lane i writes
  // 4 B at offset 256 wave + 4 i: the scale of group i % 4 of the same row.
  // Rows past N read row N-1.
  const int wrow = 16 * wave + lane / 4;
  const int wgr = (lane & 3) ^ ((wrow >> 2) & 3);
  const long wrow_g = std::min(n0 + wrow, N - 1);
  const char *wsrc0 = reinterpret_cast<const char *>(qw) + wrow_g * G * 16;
  const char *ssrc0 = reinterpret_cast<const char *>(sc) + wrow_g * G * 4;

  // pair p's raw activations (an odd G's last pair: its second group's chunks
  // re-read the first group; their products meet a zero scale)
  auto load_x = [&](unsigned char *img, int p) {
    const char *base = xtile + long(p) * 256;
    const bool one = 2 * p + 1 >= G;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t o = xoff[jj] - ((one && xhigh[jj]) ? 128u : 0u);
      const char *src = base + o;
      __builtin_amdgcn_global_load_lds(src, (lx_lds_void *)(img + 1024 * (4 * wave + jj)), 16, 0, 0);
    }
  };
  // the weights and scales of groups 4 blk .. 4 blk + 3 (groups past G re-read
  // group G-1; never used)
  auto load_ws = [&](unsigned char *wimg, unsigned char *simg, int blk) {
    const long gw = std::min(4L * blk + wgr, long(G) - 1);
    const long gs = std::min(4L * blk + (lane & 3), long(G) - 1);
    const char *wsrc = wsrc0 + gw * 16;
    __builtin_amdgcn_global_load_lds(wsrc, (lx_lds_void *)(wimg + 1024 * wave), 16, 0, 0);
    const char *ssrc = ssrc0 + gs * 4;
    __builtin_amdgcn_global_load_lds(ssrc, (lx_lds_void *)(simg + 256 * wave), 4, 0, 0);
  };

  // Split: lane (c, R) of wave w takes row 16w + c, logical chunks 4R .. 4R+3
  // (k = 16R .. 16R+15 of the pair: group R / 2, 8-blocks 2 (R % 2) and
  // 2 (R % 2) + 1 of it).
  const int srow = 16 * wave + c;
  uint32_t sread[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) sread[h] = uint32_t(srow * 256 + 16 * ((4 * R + h) ^ c));
  uint32_t swrite[2][2];  // [limb][block of the two]
#pragma unroll
  for (int l = 0; l < 2; ++l)
#pragma unroll
    for (int b = 0; b < 2; ++b) swrite[l][b] = uint32_t(srow * 256 + 16 * ((8 * l + 2 * R + b) ^ c));
  auto split = [&](const unsigned char *ximg, unsigned char *limg, float *fimg) {
    float4 v[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = *reinterpret_cast<const float4 *>(ximg + sread[h]);
    // the row's largest magnitude in the pair: over this lane's 16 values,
    // then over the row's 4 lanes (a NaN is passed over and still turns the
    // row's products to NaN)
    const float t0 = limb_absmax3(v[0].x, v[0].y, v[0].z);
    const float t1 = limb_absmax3(v[0].w, v[1].x, v[1].y);
    const float t2 = limb_absmax3(v[1].z, v[1].w, v[2].x);
    const float t3 = limb_absmax3(v[2].y, v[2].z, v[2].w);
    const float t4 = limb_absmax3(v[3].x, v[3].y, v[3].z);
    const float t5 = limb_absmax3(t0, t1, v[3].w);
    float mx = limb_absmax3(t2, t3, t4);
    mx = limb_absmax3(mx, t5, 0.0f);
    const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    mx = limb_absmax3(__uint_as_float(h32[0]), __uint_as_float(h32[1]), 0.0f);
    const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    mx = limb_absmax3(__uint_as_float(h16[0]), __uint_as_float(h16[1]), 0.0f);
    // e in [-113, 116]: 2^-e and 2^(e+11) are normal fp32 numbers, and
    // x * 2^(e+11) is exact and finite (|x| 2^e < 2^15)
    const int e = std::min(row_exponent(mx), 116);
    fimg[srow] = __int_as_float((127 - e) << 23);  // the row's 4 lanes write the same word
    const float up = __int_as_float((127 + e + 11) << 23);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float4 a = v[2 * b], d = v[2 * b + 1];  // x0..x3, x4..x7 of the block
      const float va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {d.x, d.y, d.z, d.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        limb_split2(va[i] * up, vb[i] * up, 0x1p-11f, -2048.0f, hw[i], lw[i]);
      *reinterpret_cast<uint4 *>(limg + swrite[0][b]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4 *>(limg + swrite[1][b]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  };

  // Products: limbs of row wm*32 + 16u + c, group q, block R at
  // lread[limb][q] + 4096 u; W word R of group g of row wn*64 + 16t + c at
  // wread[g] + 1024 t; its scale at sread0 + 256 t + 4 g.
  uint32_t lread[2][2];
#pragma unroll
  for (int l = 0; l < 2; ++l)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lread[l][q] = uint32_t((wm * 32 + c) * 256 + 16 * ((8 * l + 4 * q + R) ^ c));
  uint32_t wread[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) wread[g] = uint32_t((wn * 64 + c) * 64 + 16 * (g ^ ((c >> 2) & 3)) + 4 * R);
  const uint32_t sread0 = uint32_t((wn * 64 + c) * 16);
  const uint32_t fread = uint32_t((wm * 32 + 4 * R) * 4);

  float acc[2][4][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][t][r] = 0.0f;

  // pair p from its limb, factor, weight and scale images; gq0 = 2 (p % 2),
  // the pair's first group within the weight block
  auto products = [&](const unsigned char *limg, const float *fimg, const unsigned char *wimg,
                      const unsigned char *simg, int gq0, bool two) {
    float ss[2][4][4];  // the pair's sum, group scales applied, 2^-e not yet
    const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int gq = gq0 + q;
      half8_t hi[2], lo[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        hi[u] = *reinterpret_cast<const half8_t *>(limg + lread[0][q] + 4096 * u);
        lo[u] = *reinterpret_cast<const half8_t *>(limg + lread[1][q] + 4096 * u);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(wimg + wread[gq] + 1024 * t);
        const float s = *reinterpret_cast<const float *>(simg + sread0 + 256 * t + 4 * gq);
        const float sq = (q == 0 || two) ? s : 0.0f;
        const half8_t b = nibbles_to_f16(w);
        const _Float16 k2 = (_Float16)0x1p-11f;
        const half8_t b2 = b * half8_t{k2, k2, k2, k2, k2, k2, k2, k2};  // exact in fp16
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi[u], b, zero, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[u], b2, d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) ss[u][t][r] = q == 0 ? sq * d[r] : fmaf(sq, d[r], ss[u][t][r]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // 2^-e of this lane's result rows wm*32 + 16u + 4R .. +3
      const float4 fac = *reinterpret_cast<const float4 *>(
          reinterpret_cast<const unsigned char *>(fimg) + fread + 64 * u);
      const float f[4] = {fac.x, fac.y, fac.z, fac.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][t][r] = fmaf(ss[u][t][r], f[r], acc[u][t][r]);
    }
  };

  // prologue: pairs 0 and 1 copied, the first weight block, pair 0 split
  load_x(lx_x0, 0);
  if (P > 1) load_x(lx_x1, 1);
  load_ws(lx_w0, lx_s0, 0);
  lx_wait_vm0();
  lx_barrier();
  split(lx_x0, lx_l0, lx_f0);
  // Four pairs per iteration: raw, limb and factor images alternate per pair,
  // weight and scale images per two pairs (4 groups).
  for (int pb = 0; pb < P; pb += 4) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = pb + v;
      if (p < P) {
        unsigned char *xcur = (v & 1) ? lx_x1 : lx_x0;      // pair p + 2 lands here
        unsigned char *xnext = (v & 1) ? lx_x0 : lx_x1;     // pair p + 1
        unsigned char *lcur = (v & 1) ? lx_l1 : lx_l0;
        unsigned char *lnext = (v & 1) ? lx_l0 : lx_l1;
        float *fcur = (v & 1) ? lx_f1 : lx_f0;
        float *fnext = (v & 1) ? lx_f0 : lx_f1;
        unsigned char *wcur = (v & 2) ? lx_w1 : lx_w0;
        unsigned char *scur = (v & 2) ? lx_s1 : lx_s0;
        unsigned char *wnext = (v & 2) ? lx_w0 : lx_w1;
        unsigned char *snext = (v & 2) ? lx_s0 : lx_s1;
        // After the barrier: pair p + 1's copies have landed and pair p's
        // limbs are written (every wave waited for its own), and every wave is
        // past pair p - 1 (whose images the copies and limbs below replace).
        asm volatile("" ::: "memory");
        lx_wait_vm0();
        lx_wait_lgkm0();
        lx_barrier();
        // (the limbs are written before the next copies are issued: the
        // compiler waits for every copy in flight before an LDS write)
        if (p + 1 < P) split(xnext, lnext, fnext);
        if (p + 2 < P) load_x(xcur, p + 2);
        if ((v & 1) == 0 && 4 * (p / 2 + 1) < G) load_ws(wnext, snext, p / 2 + 1);
        products(lcur, fcur, wcur, scur, 2 * (v & 1), 2 * p + 1 < G);
      }
    }
  }

#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + wn * 64 + 16 * t + c;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 32 + 16 * u + 4 * R + r;
        if (m < M) Y[long(m) * N + n] = acc[u][t][r];
      }
    }
}

}  // namespace

long tile_mx_tiles(int M, int N) { return long((M + 127) / 128) * ((N + 127) / 128); }

hipError_t launch_tile_mx(const float *X, const int32_t *qweight, const float *scales, float *Y,
                          int M, int N, int K, hipStream_t stream) {
  const long tiles = tile_mx_tiles(M, N);
  if (tiles < 1 || tiles > 0x7fffffffL) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int tiles_n = (N + 127) / 128;
  hipLaunchKernelGGL(tile_mx, dim3(unsigned(tiles)), dim3(64 * kLxWaves), 0, stream, X,
                     reinterpret_cast<const uint32_t *>(qweight), scales, Y, M, N, G, tiles_n);
  return hipGetLastError();
}

}  // namespace w4a16
