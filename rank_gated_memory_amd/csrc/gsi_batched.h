// Internal layout of the batched bf16 path (gsi_batched.hip), shared with the
// host library (gsi_api.cpp).  Nothing here is part of the public ABI.
#pragma once

#include "gsi_internal.h"

namespace gsi {

constexpr int kBatchKc = 256;   // rows of V_k per split of the projection GEMM (multiple of 32)
constexpr int kMaxBatch = 4096; // tokens per batched launch (compaction list in LDS)
constexpr int kThin = 32;       // a path with at most this many tokens streams its matrix by rows

struct BArgs {
  const void *W, *V, *M, *x;
  void *y;
  float *rho;
  uint8_t *slow;
  int32_t n, d, d_out, k;
  int32_t kpad;    // k rounded up to 16 (MFMA K granularity)
  int32_t kc;      // rows of V_k per split
  int32_t splits;  // number of splits
  int32_t mode;
  float eps;
  int32_t pad_;
  const void *G;   // E = V_k^T V_k - I [k][k] bf16 (exact rho), or null
  float *part;     // [splits][n][k] partial g
  float *xxp;      // [splits][n] partial ||x||^2
  uint16_t *ghi;   // [n][kpad] bf16(g)
  uint16_t *glo;   // [n][kpad] bf16(g - hi)
  int32_t *flags;  // [n] 1 = slow
  const void *zeros;  // 256 bytes of the workspace that stay zero
};

struct BatchShape {
  int32_t kpad, kc, splits;
  uint64_t zeros_off, part_off, xxp_off, ghi_off, glo_off, flags_off, total;
};

#ifndef GSI_BPROJ_WGS
#define GSI_BPROJ_WGS 256
#endif

// Projection GEMM G = X V_k: 64 x 64 tiles of G, each split over K into
// `splits` ranges of kc rows (at least 256 workgroups in all when d allows:
// more splits cost the gate more partial rows than the extra parallelism buys).
inline BatchShape batch_shape(int n, int d, int k) {
  BatchShape b{};
  b.kpad = (k + 15) / 16 * 16;
  const int tt = (n + 63) / 64, kt = (k + 63) / 64;
  int s = (d + kBatchKc - 1) / kBatchKc;
  const int want = (GSI_BPROJ_WGS + tt * kt - 1) / (tt * kt);
  if (want > s) s = want;
  const int smax = (d + 31) / 32;
  if (s > smax) s = smax;
  int kc = (d + s - 1) / s;
  kc = (kc + 31) / 32 * 32;
  if (kc > kBatchKc) kc = kBatchKc;
  b.kc = kc;
  b.splits = (d + kc - 1) / kc;
  uint64_t off = 0;
  b.zeros_off = off;  // never written: zero since the caller zero-filled the workspace
  off += 256;
  b.part_off = off;
  off = align_up(off + (uint64_t)b.splits * n * k * 4, 256);
  b.xxp_off = off;
  off = align_up(off + (uint64_t)b.splits * n * 4, 256);
  b.ghi_off = off;
  off = align_up(off + (uint64_t)n * b.kpad * 2, 256);
  b.glo_off = off;
  off = align_up(off + (uint64_t)n * b.kpad * 2, 256);
  b.flags_off = off;
  off = align_up(off + (uint64_t)n * 4, 256);
  b.total = off;
  return b;
}

}  // namespace gsi
