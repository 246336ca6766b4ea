// Raw .qw / .sc weight files: the on-disk form of one quantized weight in the
// pages' INT4 model bundles ("The Quiet Commit: How a Single Documentation
// Edit Marks the Completion of a Major Engineering Milestone", section "The
// INT4 Milestone: From FP32 to Production-Ready Quantization"): packed int32
// words and fp32 group scales, written as bare arrays.  The files hold no
// shape or header; the reading taken here is row-major little-endian arrays
// of exactly N*K/8 int32 and N*K/32 float, with the extents from the caller.

#include "../../include/w4a16.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <sys/stat.h>

namespace {

static_assert(sizeof(int32_t) == 4 && sizeof(float) == 4, "4-byte words");

bool little_endian() {
  const uint32_t one = 1;
  unsigned char b;
  std::memcpy(&b, &one, 1);
  return b == 1;
}

int check_shape(const char *qw_path, const char *sc_path, int64_t N, int64_t K, int32_t group,
                const void *qweight, const void *scales) {
  if (!qw_path || !sc_path || !qweight || !scales) return W4A16_ERR_ARG;
  if (group != W4A16_GROUP || N < 0 || K <= 0) return W4A16_ERR_ARG;
  if (K % W4A16_GROUP != 0 || N > W4A16_MAX_N || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
  if (!little_endian()) return W4A16_ERR_IO;  // the files are little-endian words
  return W4A16_OK;
}

bool file_size_is(const char *path, uint64_t bytes) {
  struct stat st;
  if (stat(path, &st) != 0 || !S_ISREG(st.st_mode)) return false;
  return uint64_t(st.st_size) == bytes;
}

bool read_all(const char *path, void *dst, uint64_t bytes) {
  FILE *f = std::fopen(path, "rb");
  if (!f) return false;
  const size_t got = bytes ? std::fread(dst, 1, size_t(bytes), f) : 0;
  // the size was checked before; a file that changed in between is an error
  const bool at_end = std::fgetc(f) == EOF && !std::ferror(f);
  std::fclose(f);
  return got == bytes && at_end;
}

bool write_all(const char *path, const void *src, uint64_t bytes) {
  FILE *f = std::fopen(path, "wb");
  if (!f) return false;
  const size_t put = bytes ? std::fwrite(src, 1, size_t(bytes), f) : 0;
  const bool closed = std::fclose(f) == 0;
  return put == bytes && closed;
}

}  // namespace

extern "C" {

int w4a16_load_quantized(const char *qw_path, const char *sc_path, int64_t N, int64_t K,
                         int32_t group, int32_t *qweight, float *scales) {
  const int st = check_shape(qw_path, sc_path, N, K, group, qweight, scales);
  if (st != W4A16_OK) return st;
  const uint64_t bq = uint64_t(N) * uint64_t(K) / 2;
  const uint64_t bs = uint64_t(N) * uint64_t(K / W4A16_GROUP) * 4;
  if (!file_size_is(qw_path, bq) || !file_size_is(sc_path, bs)) return W4A16_ERR_IO;
  if (!read_all(qw_path, qweight, bq) || !read_all(sc_path, scales, bs)) return W4A16_ERR_IO;
  const uint64_t ns = bs / 4;
  for (uint64_t i = 0; i < ns; ++i)
    if (!std::isfinite(scales[i])) return W4A16_ERR_NONFINITE;
  return W4A16_OK;
}

int w4a16_save_quantized(const char *qw_path, const char *sc_path, int64_t N, int64_t K,
                         int32_t group, const int32_t *qweight, const float *scales) {
  const int st = check_shape(qw_path, sc_path, N, K, group, qweight, scales);
  if (st != W4A16_OK) return st;
  const uint64_t bq = uint64_t(N) * uint64_t(K) / 2;
  const uint64_t bs = uint64_t(N) * uint64_t(K / W4A16_GROUP) * 4;
  const uint64_t ns = bs / 4;
  for (uint64_t i = 0; i < ns; ++i)
    if (!std::isfinite(scales[i])) return W4A16_ERR_NONFINITE;
  if (!write_all(qw_path, qweight, bq) || !write_all(sc_path, scales, bs)) return W4A16_ERR_IO;
  return W4A16_OK;
}

}  // extern "C"
