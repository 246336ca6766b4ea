// Small-M GEMM (1 <= M <= 64 rows of X) on weights packed by
// w4a16_grouped_pack (one expert), in one contraction kernel plus, when K is
// split over workgroups, one ordered reduction.
//
// The pages' speculative decoder verifies a tree of draft tokens in one
// batch: a few dozen rows of activations against every weight matrix
// ("The Quiet Commit: How a Single Plan Update Closed Phase 3 of a Native
// DDTree Inference Engine", section "Input and Output Knowledge"), a shape
// that is memory-bound on the weights yet too wide for a GEMV.  The
// arithmetic is that of the split path (exact weight codes q - 8 in fp16, two
// fp16 limbs of each prescaled activation, fp32 accumulation, one fp32 FMA per
// group for the scale), within the tolerance of w4a16_gemm.
//
// Workgroup (column group cg, row chunk rc, K slice z): 8 waves, 2 tiles of
// 16 columns each (256 columns), up to 32 rows of X (M > 32 takes two row
// chunks, whose workgroups read the same weights and are dealt to the same
// XCD), up to 8 steps of K (a step: 4 groups, the unit of the packed layout):
//  * the X slice is copied straight from memory into LDS (global_load_lds),
//    one kilobyte per copy: one row's 32 consecutive 8-wide k blocks (a
//    segment), so each copy reads contiguous memory.  The copy lands as 32
//    pairs of 32 bytes, pair slot (j + row) mod 32 holding block j of the
//    segment, so that the 16 rows an MFMA operand read touches fall in
//    distinct LDS banks.  Then every weight and scale load of the slice is
//    issued; the copies complete first (loads retire in issue order);
//  * each row's largest magnitude within the slice (shuffle maxima per copy,
//    then across segments) gives that row's exponent for the slice, and the
//    slice is rewritten in place as fp16 limbs: a pair first holds the 8 fp32
//    values, then the 8 hi limbs and the 8 lo limbs, the hi limbs in the
//    half that held values 0..3 (the first half, or on rows whose bit 2 xor
//    bit 3 is set the second);
//  * per group, each wave reads the hi and lo fragments of every 16-row block
//    once and meets them with both of its weight tiles (2 MFMAs per pair,
//    then one FMA with the group's scale);
//  * the slice's result, with the row's power of two undone, goes to Y (one
//    slice) or to the slice's partial tile; small_reduce then adds the
//    partials in slice order (deterministic).

#include "w4a16_internal.h"
#include "gemv_common.h"
#include "limbs.h"

#include <algorithm>
#include <mutex>

namespace w4a16 {
namespace {

typedef __attribute__((address_space(3))) void sp_lds_void;

constexpr int kSpWaves = 8;
constexpr int kSpThreads = 64 * kSpWaves;
constexpr int kSpTW = 2;                          // 16-column tiles per wave
constexpr int kSpGroupTiles = kSpWaves * kSpTW;   // tiles per workgroup
constexpr int kSpTarget = 256;                    // workgroups wanted: the compute units

constexpr int kSpSteps = 8;                       // steps a workgroup stages
constexpr int kSpSegs = kSpSteps / 2;             // 32-block segments per staged row
// LDS: 16 MB rows x 16 blocks per step x 32 B, then the row exponents
__host__ __device__ constexpr int sp_image_bytes(int MB) { return 16 * MB * 16 * kSpSteps * 32; }
__host__ __device__ constexpr int sp_lds_bytes(int MB) { return sp_image_bytes(MB) + 64 * 4; }

// which half of a pair holds the hi limbs (and, before the split, values 0..3)
__device__ __forceinline__ int sp_swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// s_waitcnt with vmcnt = VM, lgkmcnt = LGKM, expcnt not waited for
template <int VM, int LGKM>
__device__ __forceinline__ void sp_waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "wait counts");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x70 | (LGKM << 8));
}

__device__ __forceinline__ void sp_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float sp_absmax(float4 a, float4 c) {
  return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
               fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
}

// MB: 16-row blocks per row chunk.  Grid: CG column groups x RC row chunks x
// S slices of sl steps (the last may be shorter); S4 steps in all.  Y when
// S == 1, else the partials [S][M][N].
template <int MB>
__global__ void __launch_bounds__(kSpThreads)
small_packed(const float *__restrict__ X, const uint4 *__restrict__ pw, const float *__restrict__ ps,
             float *__restrict__ Y, float *__restrict__ partial, int M, int N, int K, int tiles,
             int S4, int sl, int CG, int RC, int S) {
  constexpr int MR = 16 * MB;                       // staged rows
  constexpr int kChunks = kSpSegs * MR;             // 1 KB copies: (segment, row)
  constexpr int kCopies = kChunks / kSpWaves;       // per wave
  constexpr int kLoads = 2 * kSpTW * kSpSteps;      // weight and scale loads per wave
  static_assert(kChunks % kSpWaves == 0, "image shape");
  static_assert(kLoads < 64, "loads in flight");
  extern __shared__ __align__(16) unsigned char lds[];
  int *rexp = reinterpret_cast<int *>(lds + sp_image_bytes(MB));

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int cg = blockIdx.x % CG;
  const int rc = (blockIdx.x / CG) % RC;
  const int row0 = rc * MR;                         // first row of X of the chunk
  const int Mw = std::min(MR, M - row0);            // its rows inside M
  const int K8 = K / 8;
  const float *Xc = X + long(row0) * K;
  const int c16 = lane & 15;
  const int R = lane >> 4;
  const int z = int(blockIdx.x / (CG * RC));        // the slice of K
  const int st0 = z * sl;                           // first step of the slice
  const int jb0 = 16 * st0;                         // first 8-wide block of the slice
  const int jlim = std::min(16 * std::min(sl, S4 - st0), K8 - jb0);  // blocks inside slice and K

  // the X slice: copy u of wave w is chunk c = u * 8 + w (segment c / MR, row
  // c % MR); lane i writes bytes [16 i, 16 i + 16): slot i / 2, half i & 1 of
  // it, which holds block ((i / 2 - row) mod 32) of the segment, values
  // 4 h .. 4 h + 3 with h = (i & 1) ^ swz(row).  Rows past M and blocks past
  // K copy a clamped source and are zeroed at the split.
#pragma unroll
  for (int u = 0; u < kCopies; ++u) {
    const int c = u * kSpWaves + wave;
    const int seg = c / MR;
    const int r = c - seg * MR;
    const int jj = 32 * seg + (((lane >> 1) - r) & 31);
    const int h = (lane & 1) ^ sp_swz(r);
    const float *src = Xc + long(std::min(r, Mw - 1)) * K + 8 * std::min(jb0 + jj, K8 - 1) + 4 * h;
    __builtin_amdgcn_global_load_lds(src, (sp_lds_void *)(lds + c * 1024), 16, 0, 0);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // the copies are done (this wave's, then everyone's)
  sp_waitcnt<0, 15>();
  sp_barrier();

  // every weight and scale load of the slice (steps past the slice or past
  // S4 read a clamped step: their activation limbs are zero)
  int tl[kSpTW];
#pragma unroll
  for (int j = 0; j < kSpTW; ++j)
    tl[j] = std::min(cg * kSpGroupTiles + wave * kSpTW + j, tiles - 1);
  uint4 w[kSpTW][kSpSteps];
  float4 sc[kSpTW][kSpSteps];
#pragma unroll
  for (int s = 0; s < kSpSteps; ++s)
#pragma unroll
    for (int j = 0; j < kSpTW; ++j) {
      const long b = long(tl[j]) * S4 + std::min(st0 + s, S4 - 1);
      w[j][s] = load_stream16(pw + b * 64 + lane);
      sc[j][s] = *reinterpret_cast<const float4 *>(ps + (b * 16 + (lane & 15)) * 4);
    }
  __builtin_amdgcn_sched_barrier(0);

  // staging by row: the TPR threads with t / TPR = row hold its 128 pairs;
  // pair v of the row's thread k is block q = k + TPR v of the staged range
  // (segment q / 32, slot (q + row) mod 32).  The row's maximum is reduced
  // across those threads, in registers.
  constexpr int TPR = kSpThreads / MR;
  constexpr int kPV = 16 * kSpSteps / TPR;   // pairs per thread
  static_assert(kPV * TPR == 16 * kSpSteps && TPR <= 64, "staging split");
  const int sr = t / TPR;
  const int sk = t % TPR;
  const int ssw = sp_swz(sr);
  float4 va[kPV], vb[kPV];
  float mx = 0.0f;
#pragma unroll
  for (int v = 0; v < kPV; ++v) {
    const int q = sk + TPR * v;
    const unsigned char *pp = lds + ((q >> 5) * MR + sr) * 1024 + (((q & 31) + sr) & 31) * 32;
    va[v] = *reinterpret_cast<const float4 *>(pp + 16 * ssw);
    vb[v] = *reinterpret_cast<const float4 *>(pp + 16 * (ssw ^ 1));
    if (sr < Mw && q < jlim) mx = fmaxf(mx, sp_absmax(va[v], vb[v]));
  }
#pragma unroll
  for (int d = 1; d < TPR; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
  const int e = row_exponent(mx);
  if (sk == 0) rexp[sr] = e;
  // the split in place: hi limbs where values 0..3 were (each pair is read
  // and written by the same thread)
#pragma unroll
  for (int v = 0; v < kPV; ++v) {
    const int q = sk + TPR * v;
    unsigned char *pp = lds + ((q >> 5) * MR + sr) * 1024 + (((q & 31) + sr) & 31) * 32;
    half8_t hi = half8_t{0, 0, 0, 0, 0, 0, 0, 0}, lo = hi;
    if (sr < Mw && q < jlim) split_block(va[v], vb[v], e, hi, lo);
    *reinterpret_cast<half8_t *>(pp + 16 * ssw) = hi;
    *reinterpret_cast<half8_t *>(pp + 16 * (ssw ^ 1)) = lo;
  }
  sp_waitcnt<63, 0>();
  sp_barrier();

  // contraction.  A fragment of (group gg, row block i, limb L): lane
  // (c16, R) reads block j = 4 gg + R of row 16 i + c16: chunk
  // (j / 32, 16 i + c16), slot (j + 16 i + c16) mod 32, half L ^ swz(c16).
  const int sw = sp_swz(c16);
  const unsigned char *ahi = lds + c16 * 1024 + 16 * sw;
  const unsigned char *alo = lds + c16 * 1024 + 16 * (sw ^ 1);
  const int rs = R + c16;
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  floatx4 acc[kSpTW][MB];
#pragma unroll
  for (int j = 0; j < kSpTW; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = zero;
#pragma unroll
  for (int s = 0; s < kSpSteps; ++s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int gg = 4 * s + q;
      const int seg = (4 * gg) >> 5;
      half8_t ah[MB], al[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int off = (seg * MR + 16 * i) * 1024 + (((4 * gg + 16 * i + rs) & 31) << 5);
        ah[i] = *reinterpret_cast<const half8_t *>(ahi + off);
        al[i] = *reinterpret_cast<const half8_t *>(alo + off);
      }
      half8_t b[kSpTW];
      float sq[kSpTW];
#pragma unroll
      for (int j = 0; j < kSpTW; ++j) {
        const uint32_t word = q == 0 ? w[j][s].x : q == 1 ? w[j][s].y : q == 2 ? w[j][s].z : w[j][s].w;
        b[j] = nibbles_to_f16(word);
        sq[j] = q == 0 ? sc[j][s].x : q == 1 ? sc[j][s].y : q == 2 ? sc[j][s].z : sc[j][s].w;
      }
      floatx4 d[kSpTW][MB];
#pragma unroll
      for (int j = 0; j < kSpTW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
          d[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], b[j], zero, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kSpTW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
          d[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], b[j], d[j][i], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kSpTW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][i][r] = fmaf(sq[j], d[j][i][r], acc[j][i][r]);
      // the group's FMAs happen here (not sunk into the guarded stores, which
      // would keep every group's MFMA results alive), and no reads or
      // conversions of later groups are hoisted above them
#pragma unroll
      for (int j = 0; j < kSpTW; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i) asm volatile("" : "+v"(acc[j][i]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // lane (c16, R) holds rows 16 i + 4 R + r of column 16 tile + c16
  float *out = S == 1 ? Y : partial + long(z) * M * N;
#pragma unroll
  for (int j = 0; j < kSpTW; ++j) {
    const int n = (cg * kSpGroupTiles + wave * kSpTW + j) * 16 + c16;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * R + r;
        if (row < Mw && n < N)
          out[long(row0 + row) * N + n] = ldexpf(acc[j][i][r], -rexp[row]);
      }
  }
}

// Y[i] = sum over slices z = 0..S-1 of partial[z][i], added in slice order
template <bool kVec>
__global__ void __launch_bounds__(256)
small_reduce(const float *__restrict__ partial, float *__restrict__ Y, long total, int S) {
  const long i = long(blockIdx.x) * 256 + threadIdx.x;
  if constexpr (kVec) {
    const long n4 = total / 4;
    if (i >= n4) return;
    const float4 *p = reinterpret_cast<const float4 *>(partial);
    float4 v = p[i];
    for (int z0 = 1; z0 < S; z0 += 8) {
      float4 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < S) q[u] = p[long(z0 + u) * n4 + i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < S) {
          v.x += q[u].x;
          v.y += q[u].y;
          v.z += q[u].z;
          v.w += q[u].w;
        }
    }
    reinterpret_cast<float4 *>(Y)[i] = v;
  } else {
    if (i >= total) return;
    float v = partial[i];
    for (int z = 1; z < S; ++z) v += partial[long(z) * total + i];
    Y[i] = v;
  }
}

struct SmallPlan {
  int MB, RC, S4, tiles, CG, sl, S;
};

// Rows: one chunk of 16 (M <= 16) or 32 rows (M <= 32), else two chunks of
// 32.  Steps per slice: the fewest that keep the grid within one workgroup
// per compute unit, at most the 8 the image holds.
SmallPlan plan_small(int M, int N, int K) {
  SmallPlan p;
  p.MB = M <= 16 ? 1 : 2;
  p.RC = (M + 16 * p.MB - 1) / (16 * p.MB);
  p.S4 = (K / kGroup + 3) / 4;
  p.tiles = (N + 15) / 16;
  p.CG = (p.tiles + kSpGroupTiles - 1) / kSpGroupTiles;
  const long want = (long(p.S4) * p.CG * p.RC + kSpTarget - 1) / kSpTarget;
  p.sl = int(std::max(1L, std::min<long>(want, std::min(kSpSteps, p.S4))));
  p.S = (p.S4 + p.sl - 1) / p.sl;
  return p;
}

template <int MB>
void run_small(const SmallPlan &p, const float *X, const uint4 *pw, const float *ps, float *Y,
               float *partial, int M, int N, int K, hipStream_t stream) {
  const long blocks = long(p.CG) * p.RC * p.S;
  hipLaunchKernelGGL((small_packed<MB>), dim3(unsigned(blocks)), dim3(kSpThreads),
                     size_t(sp_lds_bytes(MB)), stream, X, pw, ps, Y, partial, M, N, K, p.tiles,
                     p.S4, p.sl, p.CG, p.RC, p.S);
}

}  // namespace

bool small_packed_supported(int M) { return M >= 1 && M <= 64; }

size_t small_packed_workspace_bytes(int M, int N, int K) {
  if (!small_packed_supported(M) || N <= 0 || K <= 0) return 0;
  const SmallPlan p = plan_small(M, N, K);
  return p.S > 1 ? size_t(p.S) * size_t(M) * size_t(N) * sizeof(float) : 0;
}

hipError_t launch_small_packed(const float *X, const void *packed, float *Y, int M, int N, int K,
                               void *workspace, hipStream_t stream) {
  if (!small_packed_supported(M)) return hipErrorInvalidValue;
  const SmallPlan p = plan_small(M, N, K);
  if (long(p.CG) * p.RC * p.S > 0x7fffffffL) return hipErrorInvalidValue;
  const uint4 *pw = static_cast<const uint4 *>(packed);
  const float *ps = reinterpret_cast<const float *>(pw + long(p.tiles) * p.S4 * 64);
  float *partial = static_cast<float *>(workspace);
  if (p.MB == 1)
    run_small<1>(p, X, pw, ps, Y, partial, M, N, K, stream);
  else
    run_small<2>(p, X, pw, ps, Y, partial, M, N, K, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  const long total = long(M) * N;
  if (N % 4 == 0) {
    hipLaunchKernelGGL(small_reduce<true>, dim3(unsigned((total / 4 + 255) / 256)), dim3(256), 0,
                       stream, partial, Y, total, p.S);
  } else {
    hipLaunchKernelGGL(small_reduce<false>, dim3(unsigned((total + 255) / 256)), dim3(256), 0,
                       stream, partial, Y, total, p.S);
  }
  return hipGetLastError();
}

// Fixed scratch of the allocation-free entry point: the split-K partials of
// one call.  Each device the library runs on holds its own copy for the life
// of the process.  Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol); it passes the device address
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace w4a16
