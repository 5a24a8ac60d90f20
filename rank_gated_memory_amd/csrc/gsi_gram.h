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
// g_i g_j.  Wavefront w takes rows w, w + NT/64, ...; in row r its lanes
// take the 16-byte pieces from the one holding E_rr on (shifts only, no
// division), U rows per batch with every load issued first.  Every thread
// returns the same, order-fixed sum (sh: NT/64 floats).
template <int ESIZE, int NT>
__device__ __forceinline__ float gram_quadratic(const void *E, int k, const float *g, float *sh) {
  constexpr int VW = 16 / ESIZE;
  constexpr int NW = NT / 64;
  constexpr int U = 16;
  const int n = k / VW;  // pieces per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint4 *e4 = static_cast<const uint4 *>(E);
  float acc = 0.f;
  for (int r0 = wave; r0 < k; r0 += NW * U) {
    for (int c0 = 0; c0 < n; c0 += 64) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * NW;
        const int c = r / VW + c0 + lane;  // VW is a power of two
        v[u] = (r < k && c < n) ? e4[(size_t)r * n + c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * NW;
        const int c = r / VW + c0 + lane;
        if (r < k && c < n) {
          const int col0 = c * VW;
          const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            const int col = col0 + e;
            const float ev = ESIZE == 2 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                        : __uint_as_float(w[e]);
            const float wt = col > r ? 2.f : (col == r ? 1.f : 0.f);
            sum = fmaf(wt * ev, g[col], sum);
          }
          acc = fmaf(g[r], sum, acc);
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
