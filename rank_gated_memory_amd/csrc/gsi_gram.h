// Exact residual ratio for a stored basis that is orthonormal only up to
// rounding (shared by gsi_kernels.hip and gsi_batched.hip).
//
// With g = V_k^T x, ||x - V_k g||^2 = ||x||^2 - 2 g^T g + g^T (V_k^T V_k) g
// = ||x||^2 - ||g||^2 + g^T E g for E = V_k^T V_k - I, exactly; the norm
// form sqrt(1 - ||g||^2/||x||^2) drops g^T E g, which for a bf16 basis moves
// rho by up to ~1e-3 near rho = 0.05.  gsi_prepare caches E per map.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <stdint.h>

namespace gsi {

// q = g^T E g, E [k][k] row-major with ESIZE-byte elements (2: bf16 bits,
// 4: fp32), g [k] in LDS; k a multiple of 16 / ESIZE.  E is symmetric
// (entries (i, j) and (j, i) sum the same products in the same order), so
// only its upper triangle is read: q = sum_i E_ii g_i^2 + 2 sum_{i<j} E_ij
// g_i g_j.  The triangle is walked as 64 x 64 blocks (bi <= bj, row-major
// order); wavefront w takes blocks w, w + NT/64, ...  A block is 64 rows of
// 64 / VW 16-byte pieces, so a wavefront load covers 64 / (64 / VW) whole
// row segments with every lane busy (8 lanes per 128-byte row segment for
// bf16), and 16 loads per lane are issued before any is used.  Diagonal
// blocks weight their entries 2 above the diagonal, 1 on it and 0 below.
// Every thread returns the same, order-fixed sum (sh: NT/64 floats).
template <int ESIZE, int NT>
__device__ __forceinline__ float gram_quadratic(const void *E, int k, const float *g, float *sh) {
  constexpr int VW = 16 / ESIZE;          // elements per piece
  constexpr int NW = NT / 64;
  constexpr int PB = 64 / VW;             // pieces per block row
  constexpr int RPL = 64 / PB;            // block rows per wavefront load
  constexpr int LPB = 64 / RPL;           // loads per lane per block
  constexpr int B2 = 16 / LPB;            // blocks per batch (16 loads in flight)
  const int n = k / VW;                   // pieces per row of E
  const int nb = (k + 63) / 64;
  const int nblk = nb * (nb + 1) / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane / PB, pl = lane % PB;
  const uint4 *e4 = static_cast<const uint4 *>(E);
  float acc = 0.f;
  int bi = 0, bj = 0;  // block `t` of this wavefront
  for (int s = 0; s < wave; ++s)
    if (++bj == nb) bj = ++bi;
  for (int t = wave; t < nblk; t += NW * B2) {
    int ci[B2], cj[B2];
    uint4 v[B2][LPB];
#pragma unroll
    for (int u = 0; u < B2; ++u) {
      ci[u] = bi;
      cj[u] = bj;
      const bool live = t + u * NW < nblk;
#pragma unroll
      for (int j = 0; j < LPB; ++j) {
        const int row = bi * 64 + j * RPL + rl, piece = bj * PB + pl;
        v[u][j] = (live && row < k && piece < n) ? e4[(size_t)row * n + piece] : make_uint4(0u, 0u, 0u, 0u);
      }
      for (int s = 0; s < NW; ++s)
        if (++bj == nb) bj = ++bi;
    }
#pragma unroll
    for (int u = 0; u < B2; ++u) {
      if (t + u * NW >= nblk) break;
#pragma unroll
      for (int j = 0; j < LPB; ++j) {
        const int row = ci[u] * 64 + j * RPL + rl, piece = cj[u] * PB + pl;
        if (row < k && piece < n) {
          const int col0 = piece * VW;
          const uint32_t w[4] = {v[u][j].x, v[u][j].y, v[u][j].z, v[u][j].w};
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            const int col = col0 + e;
            const float ev = ESIZE == 2 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                        : __uint_as_float(w[e]);
            const float wt = ci[u] < cj[u] ? 2.f : (col > row ? 2.f : (col == row ? 1.f : 0.f));
            sum = fmaf(wt * ev, g[col], sum);
          }
          acc = fmaf(g[row], sum, acc);
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += sh[i];
  __syncthreads();
  return t;
}

// rho from ||x||^2, ||g||^2 and the Gram term q: sqrt(max(0, xx - gg + q) / xx).
// ||x|| = 0 gives 0; a non-finite input gives NaN (the slow path).
__device__ __forceinline__ float rho_exact(float xx, float gg, float q) {
  if (!(xx <= FLT_MAX) || !(gg <= FLT_MAX) || !(fabsf(q) <= FLT_MAX)) return __builtin_nanf("");
  if (xx == 0.f) return 0.f;
  const float t = (xx - gg) + q;
  return t > 0.f ? sqrtf(t / xx) : 0.f;
}

}  // namespace gsi
