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
// 4: fp32), g [k] in LDS.  The workgroup (NT threads) streams E in 16-byte
// pieces; every thread returns the same, order-fixed sum (sh: NT/64 floats).
template <int ESIZE, int NT>
__device__ __forceinline__ float gram_quadratic(const void *E, int k, const float *g, float *sh) {
  constexpr int VW = 16 / ESIZE;
  constexpr int U = 8;
  const int pieces = k * k / VW;
  const uint4 *e4 = static_cast<const uint4 *>(E);
  float acc = 0.f;
  for (int p0 = threadIdx.x; p0 < pieces; p0 += NT * U) {
    uint4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int p = p0 + i * NT;
      v[i] = p < pieces ? e4[p] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int p = p0 + i * NT;
      if (p < pieces) {
        const int off = p * VW;
        const int row = off / k, col = off - row * k;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
          const float ev = ESIZE == 2 ? __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16))
                                      : __uint_as_float(w[e]);
          s = fmaf(ev, g[col + e], s);
        }
        acc = fmaf(g[row], s, acc);
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
