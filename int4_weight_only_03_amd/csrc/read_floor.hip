// Measurement helper, not part of the GEMM: a plain streaming read of the
// bytes a GEMM call reads (its X, qweight and scales buffers), so that a
// benchmark can time the best a single launch can do with the same bytes,
// the same buffers and the same launch cadence.  The decode path is meant to
// approach the HBM bandwidth peak ("The Quiet Commit: How a Single Plan
// Update Closed Phase 3 of a Native DDTree Inference Engine", section "Why
// This Specific Edit Matters"); what one launch of a few megabytes can reach
// on a given machine is the practical ceiling beside the 8 TB/s figure.
//
// Up to 4 segments (device pointer, byte count) are read in one launch.  Each
// thread issues L nontemporal 16-byte loads (straight-line, all in flight at
// once), strided by the grid's width in chunks so that each wave reads
// contiguous kilobytes, then folds the words with xor; the fold is stored only
// if it equals a value the data would have to be built for, so the loads
// cannot be removed and nothing else is written.

#include "w4a16_internal.h"
#include "gemv_common.h"

namespace w4a16 {
namespace {

struct Segments {
  const uint4 *p[4];
  long chunks[4];  // 16-byte chunks of each segment
  long start[4];   // first global chunk of each segment
  int n;
};

template <int L>
__global__ void __launch_bounds__(1024)
read_floor(Segments s, long total, unsigned *sink) {
  const long tid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  const long stride = long(gridDim.x) * blockDim.x;
  uint4 v[L];
#pragma unroll
  for (int u = 0; u < L; ++u) {
    long c = tid + u * stride;
    if (c >= total) c = total - 1;  // clamped: straight-line loads, always in bounds
    // the segment holding chunk c (later segments start at higher chunks)
    const uint4 *p = s.p[0];
    long off = c;
    if (s.n > 1 && c >= s.start[1]) { p = s.p[1]; off = c - s.start[1]; }
    if (s.n > 2 && c >= s.start[2]) { p = s.p[2]; off = c - s.start[2]; }
    if (s.n > 3 && c >= s.start[3]) { p = s.p[3]; off = c - s.start[3]; }
    v[u] = load_stream16(p + off);
  }
  unsigned f = 0;
#pragma unroll
  for (int u = 0; u < L; ++u) f ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (f == 0x9E3779B9u && tid == 0) sink[0] = f;
}

template <int L>
hipError_t run(const Segments &s, long total, int threads, unsigned *sink, hipStream_t stream) {
  const long per_block = long(threads) * L;
  const long blocks = (total + per_block - 1) / per_block;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_floor<L>, dim3(unsigned(blocks)), dim3(threads), 0, stream, s, total,
                     sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_read_floor(const void *const *ptrs, const long *bytes, int n, int threads,
                             int loads, unsigned *sink, hipStream_t stream) {
  Segments s{};
  long total = 0;
  for (int i = 0; i < n; ++i) {
    s.p[i] = static_cast<const uint4 *>(ptrs[i]);
    s.chunks[i] = bytes[i] / 16;
    s.start[i] = total;
    total += s.chunks[i];
  }
  s.n = n;
  if (total == 0) return hipSuccess;
  switch (loads) {
    case 1: return run<1>(s, total, threads, sink, stream);
    case 2: return run<2>(s, total, threads, sink, stream);
    case 4: return run<4>(s, total, threads, sink, stream);
    case 8: return run<8>(s, total, threads, sink, stream);
    case 16: return run<16>(s, total, threads, sink, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
