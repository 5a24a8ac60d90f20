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
  float *vw;         // [d][k] iterate (FMA path)
  float *z;          // [n][k] (FMA path)
  // matrix-core path (bf16 samples, d a multiple of 8): the fp32 operand of
  // each product as three bf16 parts (hi + mid + lo), transposed so that
  // both operands run along K
  int32_t mfma;      // 1: the products run on the matrix cores
  int32_t dp, np;    // d and n rounded up to 64 (zero padding)
  const void *zeros; // 256 bytes that stay zero
  uint16_t *vt3;     // [3][k][dp] parts of the iterate, transposed
  uint16_t *zt3;     // [3][k][np] parts of Z^T
  uint16_t *at;      // [d][np] A^T
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

// The products with A run on the matrix cores for bf16 samples whose rows
// are whole 16-byte pieces (d a multiple of 8); otherwise (fp32 samples, or
// an odd d) on fp32 FMA tiles.
inline bool calib_uses_mfma(int64_t d, int32_t dtype) { return dtype == 1 && d % 8 == 0; }

// Workspace layout (byte offsets, each 256-byte aligned): the status word
// first, then the regions of the path in use.
struct CalibLayout {
  uint64_t status, zeros, vw, z, vt3, zt3, at, y, y2, g, r, dinv, gpart, total;
  int64_t dp, np;
  bool mfma;
};

inline CalibLayout calib_layout(int64_t n, int64_t d, int64_t k, int32_t dtype) {
  auto al = [](uint64_t v) { return (v + 255) / 256 * 256; };
  CalibLayout L{};
  L.mfma = calib_uses_mfma(d, dtype);
  L.dp = (d + 63) / 64 * 64;
  L.np = (n + 63) / 64 * 64;
  uint64_t off = 0;
  L.status = off;
  off += al(256);
  if (L.mfma) {
    L.zeros = off;
    off += al(256);
    L.vt3 = off;
    off += al((uint64_t)3 * k * L.dp * 2);
    L.zt3 = off;
    off += al((uint64_t)3 * k * L.np * 2);
    L.at = off;
    off += al((uint64_t)d * L.np * 2);
  } else {
    L.vw = off;
    off += al((uint64_t)d * k * 4);
    L.z = off;
    off += al((uint64_t)n * k * 4);
  }
  L.y = off;
  off += al((uint64_t)d * k * 8);
  L.y2 = off;
  off += al((uint64_t)d * k * 8);
  L.g = off;
  off += al((uint64_t)k * k * 8);
  L.r = off;
  off += al((uint64_t)k * k * 8);
  L.dinv = off;
  off += al((uint64_t)(k + 63) / 64 * 64 * 64 * 8);
  L.gpart = off;
  off += al((uint64_t)calib_gram_splits(d, k) * k * k * 8);
  L.total = off;
  return L;
}

inline size_t calib_ws_bytes(int64_t n, int64_t d, int64_t k, int32_t dtype) {
  return calib_layout(n, d, k, dtype).total;
}

}  // namespace gsi
