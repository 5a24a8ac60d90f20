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
// g_i g_j.  The 16-byte pieces of row i from the one holding E_ii on form a
// staircase: rows of block b (rows b VW .. b VW + VW - 1) hold the pieces
// b .. n-1 (n = k / VW), so block b starts at piece VW (b n - b (b-1) / 2)
// of the flattened triangle.  The workgroup (NT threads) walks that range
// with U pieces per thread in flight; every thread returns the same,
// order-fixed sum (sh: NT/64 floats).
template <int ESIZE, int NT>
__device__ __forceinline__ float gram_quadratic(const void *E, int k, const float *g, float *sh) {
  constexpr int VW = 16 / ESIZE;
#ifndef GSI_GRAM_UNROLL
#define GSI_GRAM_UNROLL 16
#endif
  constexpr int U = GSI_GRAM_UNROLL;
  const int n = k / VW;
  const int total = VW * n * (n + 1) / 2;
  const uint4 *e4 = static_cast<const uint4 *>(E);
  const float nn = (float)(2 * n + 1);
  float acc = 0.f;
  for (int p0 = threadIdx.x; p0 < total; p0 += NT * U) {
    uint4 v[U];
    int rc[U];  // row * n + piece column
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int p = p0 + i * NT;
      int r = 0, c = 0;
      if (p < total) {
        // block b: the largest b with VW (b n - b (b-1)/2) <= p
        int b = (int)((nn - sqrtf(nn * nn - 8.f * (float)p / VW)) * 0.5f);
        b = b < 0 ? 0 : (b > n - 1 ? n - 1 : b);
        while (b > 0 && VW * (b * n - b * (b - 1) / 2) > p) --b;
        while (b < n - 1 && VW * ((b + 1) * n - (b + 1) * b / 2) <= p) ++b;
        const int q = p - VW * (b * n - b * (b - 1) / 2);
        const int len = n - b;
        r = b * VW + q / len;
        c = b + q % len;
        v[i] = e4[(size_t)r * n + c];
      } else {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
      rc[i] = p < total ? r * n + c : -1;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (rc[i] >= 0) {
        const int r = rc[i] / n, c0 = (rc[i] - r * n) * VW;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          const int col = c0 + e;
          const float ev = ESIZE == 2 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                      : __uint_as_float(w[e]);
          const float wt = col > r ? 2.f : (col == r ? 1.f : 0.f);
          s = fmaf(wt * ev, g[col], s);
        }
        acc = fmaf(g[r], s, acc);
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
