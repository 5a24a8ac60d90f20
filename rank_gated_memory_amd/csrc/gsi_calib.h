// Internal arguments of the calibration kernels (gsi_calib.hip); not ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gsi {

struct CalibArgs {
  int32_t n, d, k, dtype, iters;
  const void *A;   // [n][d] storage dtype
  const void *V0;  // [d][k] storage dtype
  void *V;         // [d][k] storage dtype
  // workspace
  uint32_t *status;  // nonzero: a Cholesky pivot was not positive
  float *vw;         // [d][k] iterate
  float *z;          // [n][k]
  double *y, *y2;    // [d][k]
  double *g, *r;     // [k][k]: Y^T Y and its Cholesky factor (upper)
  double *dinv;      // [ceil(k/64)][64][64]: inverses of R's diagonal blocks
  double *gpart;     // [calib_gram_splits(d, k)][k][k]: split partials of Y^T Y
};

// Y^T Y ([d][k] fp64) is summed over this many row ranges of Y (enough
// 64 x 64 upper-triangle tiles x ranges to fill the chip, ranges of at least
// 128 rows, partials within 64 MiB).
inline int calib_gram_splits(int64_t d, int64_t k) {
  const int64_t t = (k + 63) / 64, tu = t * (t + 1) / 2;
  int64_t s = (512 + tu - 1) / tu;
  const int64_t by_rows = d / 128, by_bytes = (int64_t(64) << 20) / (k * k * 8);
  if (s > by_rows) s = by_rows;
  if (s > by_bytes) s = by_bytes;
  return s < 1 ? 1 : (int)s;
}

// Workspace layout: status (256 B), then vw, z, y, y2, g, r, dinv, gpart,
// each 256-byte aligned.
inline size_t calib_ws_bytes(int64_t n, int64_t d, int64_t k) {
  auto al = [](uint64_t v) { return (v + 255) / 256 * 256; };
  return al(256) + al(d * k * 4) + al(n * k * 4) + 2 * al(d * k * 8) + 2 * al(k * k * 8) +
         al((k + 63) / 64 * 64 * 64 * 8) + al((uint64_t)calib_gram_splits(d, k) * k * k * 8);
}

}  // namespace gsi
