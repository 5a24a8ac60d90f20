// Basis calibration on the GPU (GSI-TS §2.3): the top-k subspace of a
// layer's activation samples by block subspace iteration
//     V <- orth(A^T (A V)),   A = [n samples][d],
// started from a random basis (cold) or from the previous layer's basis
// (the cascade the summary describes, which needs only small corrections).
//
// One sweep: Z = A V (fp32 accumulation), Y = A^T Z (fp32 accumulation,
// stored fp64), then Y = QR by CholeskyQR2 in fp64: G = Y^T Y, G = R^T R
// (Cholesky), Y <- Y R^-1, and the same once more to restore
// orthogonality to rounding.  The Q factor with a positive diagonal R is
// unique, so this is the same basis that Gram-Schmidt (DGKS) gives.
// Everything runs on the device; a Cholesky breakdown (a rank-deficient
// block) sets the workspace status word.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gsi_calib.h"

namespace gsi {
namespace {

constexpr int kCB = 256;  // threads per workgroup

template <typename T>
__device__ __forceinline__ double ld(const T *p, size_t i);
template <>
__device__ __forceinline__ double ld<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ double ld<double>(const double *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ double ld<uint16_t>(const uint16_t *p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// C[m][p] = sum_t X[t][i] Y[t][j] over t < T (AT = true: X is [T][m], the
// product is X^T Y) or C[i][j] = sum_t X[i][t] Y[t][j] (AT = false: X is
// [m][T]).  64 x 64 output block per workgroup, K in chunks of 32 through
// LDS, 4 x 4 outputs per thread, accumulator type ACC.
template <typename TX, typename TY, typename TC, typename ACC, bool AT>
__global__ void __launch_bounds__(kCB) gemm_kernel(const TX *__restrict__ X, const TY *__restrict__ Y,
                                                   TC *__restrict__ C, int m, int p, int T) {
  constexpr int KC = 32;
  __shared__ ACC Xs[KC][64 + 1];
  __shared__ ACC Ys[KC][64 + 1];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int ti = (tid >> 4) * 4, tj = (tid & 15) * 4;
  ACC acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0;
  for (int t0 = 0; t0 < T; t0 += KC) {
    for (int e = tid; e < KC * 64; e += kCB) {
      int r, c;
      if (AT) {  // X[t][i]: rows t, contiguous along i
        r = e / 64;
        c = e % 64;
        Xs[r][c] = (t0 + r < T && i0 + c < m) ? (ACC)ld(X, (size_t)(t0 + r) * m + i0 + c) : (ACC)0;
      } else {   // X[i][t]: rows i, contiguous along t
        c = e / KC;
        r = e % KC;
        Xs[r][c] = (t0 + r < T && i0 + c < m) ? (ACC)ld(X, (size_t)(i0 + c) * T + t0 + r) : (ACC)0;
      }
      const int rr = e / 64, cc = e % 64;
      Ys[rr][cc] = (t0 + rr < T && j0 + cc < p) ? (ACC)ld(Y, (size_t)(t0 + rr) * p + j0 + cc) : (ACC)0;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < KC; ++r) {
      ACC xv[4], yv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xv[a] = Xs[r][ti + a];
#pragma unroll
      for (int b = 0; b < 4; ++b) yv[b] = Ys[r][tj + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(xv[a], yv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + ti + a, j = j0 + tj + b;
      if (i < m && j < p) C[(size_t)i * p + j] = (TC)acc[a][b];
    }
}

// In place on G [k][k] (fp64, symmetric positive definite): the upper
// Cholesky factor R (G = R^T R) in the upper triangle, then R^-1 into Rinv
// (upper triangular).  One workgroup.  A pivot that keeps at most 1e-12 of
// its column's squared norm (G_jj) means the block is numerically rank
// deficient (the fp32 products leave ~1e-14 there): status <- 1.
__global__ void __launch_bounds__(kCB) chol_inv_kernel(double *G, double *Rinv, int k, uint32_t *status) {
  __shared__ double colj[1024];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    // column j of R above the diagonal is final: stage it
    for (int i = tid; i < j; i += kCB) colj[i] = G[(size_t)i * k + j];
    __syncthreads();
    if (tid == 0) {
      const double gjj = G[(size_t)j * k + j];
      double dsum = gjj;
      for (int i = 0; i < j; ++i) dsum -= colj[i] * colj[i];
      if (!(dsum > 1e-12 * gjj)) {
        s_bad = 1;
        dsum = 1.0;
      }
      G[(size_t)j * k + j] = sqrt(dsum);
    }
    __syncthreads();
    const double rjj = G[(size_t)j * k + j];
    for (int l = j + 1 + tid; l < k; l += kCB) {
      double s = G[(size_t)j * k + l];
      for (int i = 0; i < j; ++i) s -= colj[i] * G[(size_t)i * k + l];
      G[(size_t)j * k + l] = s / rjj;
    }
    __syncthreads();
  }
  // R^-1, column by column: X[j][j] = 1/R[j][j], X[i][j] = -(sum_{i<=l<j} X[i][l] R[l][j]) / R[j][j]
  for (int j = 0; j < k; ++j) {
    const double rjj = G[(size_t)j * k + j];
    for (int i = tid; i < k; i += kCB) {
      double x = 0.0;
      if (i == j) {
        x = 1.0 / rjj;
      } else if (i < j) {
        double s = 0.0;
        for (int l = i; l < j; ++l) s += Rinv[(size_t)i * k + l] * G[(size_t)l * k + j];
        x = -s / rjj;
      }
      Rinv[(size_t)i * k + j] = x;
    }
    __syncthreads();
  }
  if (tid == 0 && s_bad) *status = 1u;
}

template <typename TI, typename TO>
__global__ void __launch_bounds__(kCB) convert_kernel(const TI *in, TO *out, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kCB + threadIdx.x; i < n; i += (size_t)gridDim.x * kCB) {
    const double v = ld(in, i);
    if constexpr (sizeof(TO) == 2)
      out[i] = to_bf16((float)v);
    else
      out[i] = (TO)v;
  }
}

template <typename TX, typename TY, typename TC, typename ACC, bool AT>
void gemm(const TX *X, const TY *Y, TC *C, int m, int p, int T, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<TX, TY, TC, ACC, AT>), dim3((m + 63) / 64, (p + 63) / 64), dim3(kCB), 0, s, X,
                     Y, C, m, p, T);
}

template <typename TI, typename TO>
void convert(const TI *in, TO *out, size_t n, hipStream_t s) {
  size_t blocks = (n + kCB - 1) / kCB;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL((convert_kernel<TI, TO>), dim3((unsigned)blocks), dim3(kCB), 0, s, in, out, n);
}

// Q <- the Q factor of Y ([d][k] fp64), one CholeskyQR pass.
void cholqr_pass(const double *Y, double *Q, double *G, double *Rinv, int d, int k, uint32_t *status,
                 hipStream_t s) {
  gemm<double, double, double, double, true>(Y, Y, G, k, k, d, s);     // G = Y^T Y
  hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kCB), 0, s, G, Rinv, k, status);
  gemm<double, double, double, double, false>(Y, Rinv, Q, d, k, k, s);  // Q = Y R^-1
}

template <typename T>
hipError_t run(const CalibArgs &c, hipStream_t s) {
  const T *A = static_cast<const T *>(c.A);
  convert(static_cast<const T *>(c.V0), c.vw, (size_t)c.d * c.k, s);
  for (int it = 0; it < c.iters; ++it) {
    gemm<T, float, float, float, false>(A, c.vw, c.z, c.n, c.k, c.d, s);    // Z = A V      [n][k]
    gemm<T, float, double, float, true>(A, c.z, c.y, c.d, c.k, c.n, s);     // Y = A^T Z    [d][k]
    cholqr_pass(c.y, c.y2, c.g, c.rinv, c.d, c.k, c.status, s);  // y2 = Q(y)
    cholqr_pass(c.y2, c.y, c.g, c.rinv, c.d, c.k, c.status, s);  // y = Q(y2): orthogonal to rounding
    if (it + 1 < c.iters) convert(c.y, c.vw, (size_t)c.d * c.k, s);
  }
  if (c.iters == 0)
    convert(static_cast<const T *>(c.V0), static_cast<T *>(c.V), (size_t)c.d * c.k, s);
  else
    convert(c.y, static_cast<T *>(c.V), (size_t)c.d * c.k, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs &c, hipStream_t s) {
  if (c.dtype == 0) return run<float>(c, s);
  return run<uint16_t>(c, s);
}

}  // namespace gsi
