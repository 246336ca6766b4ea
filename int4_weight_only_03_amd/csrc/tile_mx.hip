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
// Pipeline, per pair of groups p (one s_barrier each).  Three LDS images each
// hold one pair's 128 activation rows, first raw and then, split in place, as
// limbs; two hold a pair's fp16 weight codes.  In iteration p every wave
//   * issues the copies of pair p + 2's raw activations and scales (direct
//     copies into the image pair p - 1 used) and loads pair p + 2's weight
//     words (8 bytes per lane) into registers;
//   * reads pair p's limbs, codes, scales and factors 2^-e, and pair p + 1's
//     raw activations of its own 16 rows (copied by itself);
//   * converts pair p + 1's weight words (loaded one pair earlier) into codes
//     and splits pair p + 1 (the rows' pair maximum over 4 lanes, the
//     exponent, the limbs, written over the raw values) while it runs pair
//     p's matrix instructions.
// Every copy and load of an iteration is waited for before the next one's
// barrier, one iteration after it was issued.  Images are separate __shared__
// objects.
//
// Repacked weights (kPacked: the layout w4a16_repack writes, 16-row tiles by
// 4-group steps, each 16-byte chunk one word of the step's 4 groups of one
// row): thread t takes chunk t % 64 of tile t / 64 of the workgroup's 8, so
// one 16-byte load per thread brings two pairs' words (every other
// iteration), and the scales of a pair come from the step's 256-byte block.
// The layout pads rows to 16 and groups to 4 with code 0 and scale 0, so no
// weight or scale read needs a clamp.

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
// Direct copy global -> LDS of 16 (or 4) bytes per lane: lane i writes at
// lds + 16 i (4 i).  Written as asm so that the compiler does not track the
// copies: it cannot tell their target images from the ones being read and
// would wait for every copy in flight before each LDS access; the kernel's own
// vmcnt waits order the copies.  The LDS address is wave-uniform (m0).
__device__ __forceinline__ void lx_copy16(const void *src, const void *lds) {
  const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((const lx_lds_void *)lds));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(a) : "memory", "m0");
}
__device__ __forceinline__ void lx_copy4(const void *src, const void *lds) {
  const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((const lx_lds_void *)lds));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 1\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(a) : "memory", "m0");
}
// Workgroup barrier without the release fence of __syncthreads() (which would
// wait for the next pairs' copies as well).
__device__ __forceinline__ void lx_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// kPacked: qw points at the repacked chunks and sc at the repacked scales;
// S4 = 4-group steps per tile, T16 = 16-row tiles.
template <bool kPacked>
__global__ void __launch_bounds__(64 * kLxWaves)
tile_mx(const float *__restrict__ X, const uint32_t *__restrict__ qw,
        const float *__restrict__ sc, float *__restrict__ Y, int M, int N, int G, int tiles_n,
        int S4, int T16) {
  // A pair's activations: row r at 256 r.  Raw: logical chunk L (k = 4L..4L+3
  // of the pair) at physical chunk L ^ (r % 16).  Limbs: logical chunk
  // 8 limb + 4 q + b (limb 0 = hi, 1 = lo; group q; k = 8b .. 8b+7 of the
  // group, in the order the nibble conversion produces) at physical chunk
  // (8 limb + 4 q + b) ^ (r % 16).  Pair p lives in image p % 3.
  __shared__ __align__(16) unsigned char lx_a0[128 * 256];
  __shared__ __align__(16) unsigned char lx_a1[128 * 256];
  __shared__ __align__(16) unsigned char lx_a2[128 * 256];
  // a pair's fp16 codes q - 8: W row n at 128 n, word R of group q (8 codes,
  // in the nibble conversion's order) at chunk (4 q + R) ^ ((n / 2) % 8);
  // pair p in image p % 2
  __shared__ __align__(16) unsigned char lx_c0[128 * 128];
  __shared__ __align__(16) unsigned char lx_c1[128 * 128];
  // a pair's scales: row n at 8 n; pair p in image p % 3
  __shared__ __align__(16) unsigned char lx_s0[128 * 8];
  __shared__ __align__(16) unsigned char lx_s1[128 * 8];
  __shared__ __align__(16) unsigned char lx_s2[128 * 8];
  // 2^-e of a pair, per row; pair p in image p % 2
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
  // Scale copy (waves 0-3): lane i of wave w writes 4 B at 256 w + 4 i: row
  // 32 w + i/2, group i % 2 of the pair.  Rows past N read row N-1 (public
  // layout) or the padded rows of the last tile (repacked).
  const int srow_c = 32 * (wave & 3) + lane / 2;
  const char *ssrc0;
  if constexpr (kPacked) {
    // the step's block of tile n / 16: float (b * 16 + n % 16) * 4 + q
    const int tl = std::min((n0 + srow_c) >> 4, T16 - 1);
    ssrc0 = reinterpret_cast<const char *>(sc) + (long(tl) * S4 * 64 + ((n0 + srow_c) & 15) * 4) * 4;
  } else {
    ssrc0 = reinterpret_cast<const char *>(sc) + long(std::min(n0 + srow_c, N - 1)) * G * 4;
  }
  // Weight words.  Public layout: thread t loads 8 B of W row t / 4: words
  // 2 (t % 4) and 2 (t % 4) + 1 of the pair (group (t % 4) / 2, words
  // R = 2 (t % 2), +1).  Repacked: thread t loads the 16-byte chunk
  // c + 16 R = t % 64 of tile t / 64: word R of the step's 4 groups of row
  // 16 (t / 64) + c, i.e. word R of both groups of two pairs.
  const int tid = int(threadIdx.x);
  const int cn = kPacked ? 16 * (tid >> 6) + (tid & 15) : tid >> 2;
  const int ch = tid & 3, cq = ch >> 1;
  const char *wsrc0;
  uint32_t cwrite[2];
  if constexpr (kPacked) {
    const int tl = std::min((n0 >> 4) + (tid >> 6), T16 - 1);
    wsrc0 = reinterpret_cast<const char *>(qw) + (long(tl) * S4 * 64 + (tid & 63)) * 16;
    const int Rw = (tid >> 4) & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) cwrite[i] = uint32_t(cn * 128 + 16 * ((4 * i + Rw) ^ ((cn >> 1) & 7)));
  } else {
    wsrc0 = reinterpret_cast<const char *>(qw) + long(std::min(n0 + cn, N - 1)) * G * 16 + 8 * ch;
#pragma unroll
    for (int i = 0; i < 2; ++i) cwrite[i] = uint32_t(cn * 128 + 16 * ((2 * ch + i) ^ ((cn >> 1) & 7)));
  }

  // pair p's raw activations and scales (an odd G's last pair: its second
  // group's chunks re-read the first group; their products meet a zero scale)
  auto copy_pair = [&](unsigned char *img, unsigned char *simg, int p) {
    const char *base = xtile + long(p) * 256;
    const bool one = 2 * p + 1 >= G;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t o = xoff[jj] - ((one && xhigh[jj]) ? 128u : 0u);
      lx_copy16(base + o, img + 1024 * (4 * wave + jj));
    }
    if (wave < 4) {
      if constexpr (kPacked) {
        // step p / 2 of the tile's blocks, groups 2 (p % 2) + (lane % 2)
        lx_copy4(ssrc0 + (long(p >> 1) * 64 + 2 * (p & 1) + (lane & 1)) * 4, simg + 256 * wave);
      } else {
        const int g = std::min(2 * p + (lane & 1), G - 1);
        lx_copy4(ssrc0 + long(g) * 4, simg + 256 * wave);
      }
    }
  };
  auto load_w = [&](int p) -> uint2 {
    const long off = long(p) * 32 - ((2 * p + 1 >= G && cq) ? 16 : 0);
    return *reinterpret_cast<const uint2 *>(wsrc0 + off);
  };
  // repacked: the words of pairs 2 s' and 2 s' + 1 (step s')
  auto load_chunk = [&](int sp) -> uint4 {
    return *reinterpret_cast<const uint4 *>(wsrc0 + long(sp) * 1024);
  };
  auto convert_w = [&](uint2 w, unsigned char *cimg) {
    const half8_t b0 = nibbles_to_f16(w.x), b1 = nibbles_to_f16(w.y);
    *reinterpret_cast<half8_t *>(cimg + cwrite[0]) = b0;
    *reinterpret_cast<half8_t *>(cimg + cwrite[1]) = b1;
  };

  // Split: lane (c, R) of wave w takes row 16w + c, logical chunks 4R .. 4R+3
  // (k = 16R .. 16R+15 of the pair: group R / 2, 8-blocks 2 (R % 2) and
  // 2 (R % 2) + 1 of it).  Every lane of a row has read its raw chunks before
  // any writes limbs (the row maximum needs all four), and no other wave
  // touches the row, so the limbs can replace the raw values.
  const int srow = 16 * wave + c;
  uint32_t sread[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) sread[h] = uint32_t(srow * 256 + 16 * ((4 * R + h) ^ c));
  uint32_t swrite[2][2];  // [limb][block of the two]
#pragma unroll
  for (int l = 0; l < 2; ++l)
#pragma unroll
    for (int b = 0; b < 2; ++b) swrite[l][b] = uint32_t(srow * 256 + 16 * ((8 * l + 2 * R + b) ^ c));
  auto split_read = [&](const unsigned char *img, float4 (&v)[4]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) v[h] = *reinterpret_cast<const float4 *>(img + sread[h]);
  };
  auto split_write = [&](const float4 (&v)[4], unsigned char *img, float *fimg) {
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
      *reinterpret_cast<uint4 *>(img + swrite[0][b]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4 *>(img + swrite[1][b]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  };

  // Products: limbs of row wm*32 + 16u + c, group q, block R at
  // lread[limb][q] + 4096 u; codes of W row wn*64 + 16t + c, word R of group
  // q at cread[q] + 2048 t; its scale at sread0 + 128 t + 4 q; the factors of
  // result rows wm*32 + 16u + 4R .. +3 at fread + 64 u.
  uint32_t lread[2][2];
#pragma unroll
  for (int l = 0; l < 2; ++l)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lread[l][q] = uint32_t((wm * 32 + c) * 256 + 16 * ((8 * l + 4 * q + R) ^ c));
  uint32_t cread[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int n = wn * 64 + c;
    cread[q] = uint32_t(n * 128 + 16 * ((4 * q + R) ^ ((n >> 1) & 7)));
  }
  const uint32_t sread0 = uint32_t((wn * 64 + c) * 8);
  const uint32_t fread = uint32_t((wm * 32 + 4 * R) * 4);

  struct Ops {
    half8_t hi[2][2], lo[2][2];  // [q][u]
    half8_t b[2][4];             // [q][t]
    float s[2][4];
    float4 fac[2];
  };
  auto products_read = [&](const unsigned char *img, const unsigned char *cimg,
                           const unsigned char *simg, const float *fimg, Ops &o) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        o.hi[q][u] = *reinterpret_cast<const half8_t *>(img + lread[0][q] + 4096 * u);
        o.lo[q][u] = *reinterpret_cast<const half8_t *>(img + lread[1][q] + 4096 * u);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o.b[q][t] = *reinterpret_cast<const half8_t *>(cimg + cread[q] + 2048 * t);
        o.s[q][t] = *reinterpret_cast<const float *>(simg + sread0 + 128 * t + 4 * q);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      o.fac[u] = *reinterpret_cast<const float4 *>(
          reinterpret_cast<const unsigned char *>(fimg) + fread + 64 * u);
  };

  float acc[2][4][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][t][r] = 0.0f;

  auto products = [&](const Ops &o, bool two) {
    float ss[2][4][4];  // the pair's sum, group scales applied, 2^-e not yet
    const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float sq = (q == 0 || two) ? o.s[q][t] : 0.0f;
        const half8_t b = o.b[q][t];
        const _Float16 k2 = (_Float16)0x1p-11f;
        const half8_t b2 = b * half8_t{k2, k2, k2, k2, k2, k2, k2, k2};  // exact in fp16
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.hi[q][u], b, zero, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.lo[q][u], b2, d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) ss[u][t][r] = q == 0 ? sq * d[r] : fmaf(sq, d[r], ss[u][t][r]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float f[4] = {o.fac[u].x, o.fac[u].y, o.fac[u].z, o.fac[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][t][r] = fmaf(ss[u][t][r], f[r], acc[u][t][r]);
    }
  };

  // prologue: pairs 0 and 1 copied and their weight words loaded; pair 0's
  // codes converted and its activations split
  copy_pair(lx_a0, lx_s0, 0);
  uint2 wnext, wlater;
  uint2 whalf = {0u, 0u};  // repacked: pair p + 3's words, loaded with pair p + 2's
  if constexpr (kPacked) {
    const uint4 c0 = load_chunk(0);
    wnext = make_uint2(c0.x, c0.y);
    wlater = make_uint2(c0.z, c0.w);
    if (P > 1) copy_pair(lx_a1, lx_s1, 1);
  } else {
    wnext = load_w(0);
    wlater = wnext;
    if (P > 1) {
      copy_pair(lx_a1, lx_s1, 1);
      wlater = load_w(1);
    }
  }
  lx_wait_vm0();
  {
    float4 v[4];
    split_read(lx_a0, v);  // this wave's own copies
    convert_w(wnext, lx_c0);
    split_write(v, lx_a0, lx_f0);
  }
  wnext = wlater;
  // Six pairs per iteration (activation and scale images by p % 3, codes and
  // factors by p % 2).
  for (int pb = 0; pb < P; pb += 6) {
#pragma unroll
    for (int v = 0; v < 6; ++v) {
      const int p = pb + v;
      if (p < P) {
        const int i3 = v % 3;
        unsigned char *acur = i3 == 0 ? lx_a0 : i3 == 1 ? lx_a1 : lx_a2;
        unsigned char *anext = i3 == 0 ? lx_a1 : i3 == 1 ? lx_a2 : lx_a0;
        unsigned char *afree = i3 == 0 ? lx_a2 : i3 == 1 ? lx_a0 : lx_a1;
        unsigned char *scur = i3 == 0 ? lx_s0 : i3 == 1 ? lx_s1 : lx_s2;
        unsigned char *sfree = i3 == 0 ? lx_s2 : i3 == 1 ? lx_s0 : lx_s1;
        unsigned char *ccur = (v & 1) ? lx_c1 : lx_c0;
        unsigned char *cnext = (v & 1) ? lx_c0 : lx_c1;
        float *fcur = (v & 1) ? lx_f1 : lx_f0;
        float *fnext = (v & 1) ? lx_f0 : lx_f1;
        // Every copy and load issued one pair ago has landed (pair p + 1's
        // activations, scales and weight words); after the barrier every
        // wave's have, pair p's limbs and codes are written, and every wave
        // is past pair p - 1 (whose images are reused below).
        asm volatile("" ::: "memory");
        lx_wait_vm0();
        lx_wait_lgkm0();
        lx_barrier();
        const uint2 wcur = wnext;  // pair p + 1's weight words
        if (p + 2 < P) {
          copy_pair(afree, sfree, p + 2);
          if constexpr (kPacked) {
            if ((v & 1) == 0) {  // p even: pairs p + 2 and p + 3 in one chunk
              const uint4 c = load_chunk((p + 2) >> 1);
              wnext = make_uint2(c.x, c.y);
              whalf = make_uint2(c.z, c.w);
            } else {
              wnext = whalf;
            }
          } else {
            wnext = load_w(p + 2);
          }
        }
        Ops o;
        products_read(acur, ccur, scur, fcur, o);
        const bool more = p + 1 < P;
        float4 xv[4];
        if (more) split_read(anext, xv);
        if (more) convert_w(wcur, cnext);
        products(o, 2 * p + 1 < G);
        if (more) split_write(xv, anext, fnext);
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

long tile_mx_tiles(int M, int N) { return ((long(M) + 127) / 128) * ((long(N) + 127) / 128); }

hipError_t launch_tile_mx(const float *X, const int32_t *qweight, const float *scales, float *Y,
                          int M, int N, int K, hipStream_t stream) {
  const long tiles = tile_mx_tiles(M, N);
  if (tiles < 1 || tiles > 0x7fffffffL) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int tiles_n = (N + 127) / 128;
  hipLaunchKernelGGL(tile_mx<false>, dim3(unsigned(tiles)), dim3(64 * kLxWaves), 0, stream, X,
                     reinterpret_cast<const uint32_t *>(qweight), scales, Y, M, N, G, tiles_n, 0, 0);
  return hipGetLastError();
}

hipError_t launch_tile_mx_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                                 hipStream_t stream) {
  const long tiles = tile_mx_tiles(M, N);
  if (tiles < 1 || tiles > 0x7fffffffL) return hipErrorInvalidValue;
  const int G = K / kGroup;
  const int tiles_n = (N + 127) / 128;
  const int T16 = (N + 15) / 16, S4 = (G + 3) / 4;
  const unsigned char *pk = static_cast<const unsigned char *>(packed);
  const float *psc = reinterpret_cast<const float *>(pk + size_t(T16) * S4 * 1024);
  hipLaunchKernelGGL(tile_mx<true>, dim3(unsigned(tiles)), dim3(64 * kLxWaves), 0, stream, X,
                     reinterpret_cast<const uint32_t *>(pk), psc, Y, M, N, G, tiles_n, S4, T16);
  return hipGetLastError();
}

}  // namespace w4a16
