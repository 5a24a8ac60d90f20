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
};

// Workspace layout: status (256 B), then vw, z, y, y2, g, r, dinv, each 256-byte aligned.
inline size_t calib_ws_bytes(int64_t n, int64_t d, int64_t k) {
  auto al = [](uint64_t v) { return (v + 255) / 256 * 256; };
  return al(256) + al(d * k * 4) + al(n * k * 4) + 2 * al(d * k * 8) + 2 * al(k * k * 8) +
         al((k + 63) / 64 * 64 * 64 * 8);
}

}  // namespace gsi
