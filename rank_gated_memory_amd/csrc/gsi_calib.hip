// Basis calibration on the GPU (GSI-TS §2.3): the top-k subspace of a
// layer's activation samples by block subspace iteration
//     V <- orth(A^T (A V)),   A = [n samples][d],
// started from a random basis (cold) or from the previous layer's basis
// (the cascade the summary describes, which needs only small corrections).
//
// One sweep: Z = A V (fp32 accumulation), Y = A^T Z (fp32 accumulation,
// stored fp64), then Y = QR by CholeskyQR2 in fp64: G = Y^T Y, G = R^T R
// (blocked Cholesky), Y <- Y R^-1 (blocked substitution), and the same once
// more to restore orthogonality to rounding.  The Q factor with a positive
// diagonal R is unique, so this is the same basis that Gram-Schmidt (DGKS)
// gives.  With bf16 samples the two products run on the matrix cores (the
// fp32 operand as three bf16 parts, see mgemm_kernel), otherwise on fp32 FMA
// tiles.  Everything runs on the device; a Cholesky breakdown (a
// rank-deficient block) sets the workspace status word.
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

// ---------------------------------------------------------------------------
// Matrix-core products for bf16 samples.  Every product with A has one bf16
// operand (A or A^T) and one fp32 operand (the iterate V, or Z = A V).  The
// fp32 operand is carried as three bf16 parts hi + mid + lo (each the
// rounding of what the previous ones leave, so together they hold its 24
// significant bits), and the product is the sum of the three bf16 products
// accumulated in fp32 by v_mfma_f32_32x32x16_bf16: the same fp32-accumulated
// product as the FMA tiles, at the matrix cores' rate.  Both operands are
// stored along K (rows of 16-byte pieces), padded with zeros to 64.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// v = hi + mid + lo to about 2^-24 |v| (each part rounds the remainder).
__device__ __forceinline__ void split3(float v, uint16_t *p) {
  const uint16_t hi = to_bf16(v);
  const float r1 = v - from_bf16(hi);
  const uint16_t mid = to_bf16(r1);
  p[0] = hi;
  p[1] = mid;
  p[2] = to_bf16(r1 - from_bf16(mid));
}

// At[i][s] = A[s][i] for s < n, zero for n <= s < np (64 x 64 tiles through
// LDS); workgroup (0, 0) also clears the 256-byte zero block.
__global__ void __launch_bounds__(kCB) transpose_pad_kernel(const uint16_t *__restrict__ A, uint16_t *__restrict__ At,
                                                            uint32_t *zeros, int n, int d, int np) {
  __shared__ uint16_t T[64][66];
  const int tid = threadIdx.x;
  const int s0 = blockIdx.x * 64, i0 = blockIdx.y * 64;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid < 64) zeros[tid] = 0u;
  for (int e = tid; e < 64 * 64; e += kCB) {
    const int s = e / 64, i = e % 64;
    T[s][i] = (s0 + s < n && i0 + i < d) ? A[(size_t)(s0 + s) * d + i0 + i] : (uint16_t)0;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += kCB) {
    const int i = e / 64, s = e % 64;
    if (i0 + i < d) At[(size_t)(i0 + i) * np + s0 + s] = T[s][i];
  }
}

// parts[p][j][i] = part p of (float)Y[i][j] for i < d, zero for d <= i < dp
// (Y [d][k], 64 x 64 tiles through LDS).
template <typename TY>
__global__ void __launch_bounds__(kCB) split_t_kernel(const TY *__restrict__ Y, uint16_t *__restrict__ parts, int d,
                                                      int k, int dp) {
  __shared__ float T[64][65];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  for (int e = tid; e < 64 * 64; e += kCB) {
    const int i = e / 64, j = e % 64;
    T[i][j] = (i0 + i < d && j0 + j < k) ? (float)ld(Y, (size_t)(i0 + i) * k + j0 + j) : 0.f;
  }
  __syncthreads();
  const size_t ps = (size_t)k * dp;
  for (int e = tid; e < 64 * 64; e += kCB) {
    const int j = e / 64, i = e % 64;
    if (j0 + j < k) {
      uint16_t p[3];
      split3(T[i][j], p);
      const size_t o = (size_t)(j0 + j) * dp + i0 + i;
      parts[o] = p[0];
      parts[ps + o] = p[1];
      parts[2 * ps + o] = p[2];
    }
  }
}

// C[i][j] = sum_t P[i][t] Q[j][t], t < K: P rows i < M (NP parts, part
// stride sp), Q rows j < N (NQ parts, part stride sq), rows along K with
// strides ldp, ldq (multiples of 8).  OUT 0: C as three bf16 parts
// [3][M][ldc] (part stride sc), columns up to ldc written (zero past N);
// OUT 1: C fp64 [M][ldc], columns below N; OUT 2: the fp32 partial sum over
// blockIdx.z's share of the K chunks, [gridDim.z][M][ldc], columns up to
// ldc.
struct MGemm {
  const uint16_t *P, *Q;
  void *C;
  const u32x4_t *zero;
  int M, N, K, ldp, ldq, ldc;
  size_t sp, sq, sc;
};

constexpr int kMRow = 9;  // 16-byte pieces per staged 64-wide K row, padded (bank spread)
// 64 x 64 tile of C per workgroup, four wavefronts of 32 x 32; K in chunks of
// 64 through double-buffered LDS.  The loads run DEPTH chunks ahead, in a
// ring of register stages: the stage just written to LDS is refilled with
// chunk ch + DEPTH.  A chunk's multiplications are far shorter than the
// latency of its loads, which a deeper ring covers where the operand
// traffic leaves room (Y = A^T Z: 113 -> 100 us per launch on average at
// DEPTH 3); Z^T = V^T A^T re-reads the three parts of V^T once per 64
// samples and gains nothing from it.  Pieces outside the operands read the
// zero block.
template <int NP, int NQ, int OUT, int DEPTH>
__global__ void __launch_bounds__(kCB) mgemm_kernel(MGemm g) {
  __shared__ u32x4_t Ps[2][NP][64 * kMRow];
  __shared__ u32x4_t Qs[2][NQ][64 * kMRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int wi = wave >> 1, wj = wave & 1;
  const u32x4_t *zero = g.zero + (lane & 15);
  u32x4_t pr[DEPTH][NP][2], qr[DEPTH][NQ][2];
  auto load = [&](u32x4_t (&ps)[NP][2], u32x4_t (&qs)[NQ][2], int kk) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = tid + h * kCB, r = v >> 3, c = kk + (v & 7) * 8;
      const bool kok = c < g.K;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        ps[p][h] = *((kok && i0 + r < g.M)
                         ? reinterpret_cast<const u32x4_t *>(g.P + p * g.sp + (size_t)(i0 + r) * g.ldp + c)
                         : zero);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        qs[q][h] = *((kok && j0 + r < g.N)
                         ? reinterpret_cast<const u32x4_t *>(g.Q + q * g.sq + (size_t)(j0 + r) * g.ldq + c)
                         : zero);
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const int nch_all = (g.K + 63) / 64, per = (nch_all + gridDim.z - 1) / gridDim.z;
  const int cb = blockIdx.z * per;  // first K chunk of this workgroup
  const int nch = max(0, min(per, nch_all - cb));
#pragma unroll
  for (int st = 0; st < DEPTH; ++st)
    if (st < nch) load(pr[st], qr[st], (cb + st) * 64);
  for (int ch0 = 0; ch0 < nch; ch0 += DEPTH) {
#pragma unroll
    for (int st = 0; st < DEPTH; ++st) {
      const int ch = ch0 + st;
      if (ch >= nch) break;  // the same for every thread of the workgroup
      const int b = ch & 1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int v = tid + h * kCB, r = v >> 3, c = v & 7;
#pragma unroll
        for (int p = 0; p < NP; ++p) Ps[b][p][r * kMRow + c] = pr[st][p][h];
#pragma unroll
        for (int q = 0; q < NQ; ++q) Qs[b][q][r * kMRow + c] = qr[st][q][h];
      }
      if (ch + DEPTH < nch) load(pr[st], qr[st], (cb + ch + DEPTH) * 64);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int pc = ks * 2 + (lane >> 5);
        bf16x8_t a[NP], bq[NQ];
#pragma unroll
        for (int p = 0; p < NP; ++p)
          a[p] = __builtin_bit_cast(bf16x8_t, Ps[b][p][(32 * wi + (lane & 31)) * kMRow + pc]);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          bq[q] = __builtin_bit_cast(bf16x8_t, Qs[b][q][(32 * wj + (lane & 31)) * kMRow + pc]);
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int q = 0; q < NQ; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p], bq[q], acc, 0, 0, 0);
      }
    }
  }
  // accumulator e of lane l: C[8 (e / 4) + 4 (l / 32) + e % 4][l % 32] of the wavefront's block
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int i = i0 + 32 * wi + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
    const int j = j0 + 32 * wj + (lane & 31);
    if (i >= g.M) continue;
    if (OUT == 0) {
      if (j < g.ldc) {
        uint16_t pt[3];
        split3(acc[e], pt);
        uint16_t *C = static_cast<uint16_t *>(g.C) + (size_t)i * g.ldc + j;
        C[0] = pt[0];
        C[g.sc] = pt[1];
        C[2 * g.sc] = pt[2];
      }
    } else if (OUT == 2) {
      if (j < g.ldc) static_cast<float *>(g.C)[((size_t)blockIdx.z * g.M + i) * g.ldc + j] = acc[e];
    } else if (j < g.N) {
      static_cast<double *>(g.C)[(size_t)i * g.ldc + j] = (double)acc[e];
    }
  }
}

// Blocked fp64 factorisation, 64 x 64 tiles in LDS (rows padded to 65).
constexpr int kNb = 64;
constexpr int kLd = kNb + 1;



// dst[r][c] = M[(r0 + r) * ld + c0 + c] for r < nr, c < nc, zero elsewhere.
// Every load of the tile is issued before the first LDS store.
constexpr int kTileLoads = kNb * kNb / kCB;
__device__ __forceinline__ void load_tile(double (*dst)[kLd], const double *M, size_t ld, int r0, int c0,
                                          int nr, int nc) {
  double v[kTileLoads];
#pragma unroll
  for (int q = 0; q < kTileLoads; ++q) {
    const int e = threadIdx.x + q * kCB;
    const int r = e / kNb, c = e % kNb;
    v[q] = (r < nr && c < nc) ? M[(size_t)(r0 + r) * ld + c0 + c] : 0.0;
  }
#pragma unroll
  for (int q = 0; q < kTileLoads; ++q) {
    const int e = threadIdx.x + q * kCB;
    dst[e / kNb][e % kNb] = v[q];
  }
}

// Two tiles at once (all 32 loads in flight).
__device__ __forceinline__ void load_tiles2(double (*da)[kLd], const double *Ma, size_t lda, int ra, int ca,
                                            int nra, int nca, double (*db)[kLd], const double *Mb, size_t ldb,
                                            int rb, int cb, int nrb, int ncb) {
  double va[kTileLoads], vb[kTileLoads];
#pragma unroll
  for (int q = 0; q < kTileLoads; ++q) {
    const int e = threadIdx.x + q * kCB;
    const int r = e / kNb, c = e % kNb;
    va[q] = (r < nra && c < nca) ? Ma[(size_t)(ra + r) * lda + ca + c] : 0.0;
    vb[q] = (r < nrb && c < ncb) ? Mb[(size_t)(rb + r) * ldb + cb + c] : 0.0;
  }
#pragma unroll
  for (int q = 0; q < kTileLoads; ++q) {
    const int e = threadIdx.x + q * kCB;
    da[e / kNb][e % kNb] = va[q];
    db[e / kNb][e % kNb] = vb[q];
  }
}

// Products of 64 x 64 fp64 tiles in LDS on the matrix cores
// (v_mfma_f64_16x16x4f64: each operand value a lane loads from LDS serves 16
// products, against 2 per value for 4 x 4 register tiles of FMAs, which left
// these kernels bound by LDS bandwidth).  Wavefront w owns the 32 x 32 block
// at rows 32 (w / 2), columns 32 (w % 2), as 2 x 2 accumulators of 16 x 16.
// Lane layout (checked on the device): lane l holds A[l % 16][l / 16] and
// B[l / 16][l % 16] of a 16 x 4 by 4 x 16 step, and element e of its
// accumulator is C[4 e + l / 16][l % 16].
typedef double f64x4_t __attribute__((ext_vector_type(4)));
struct Blk {
  f64x4_t c[2][2];
};
__device__ __forceinline__ int blk_r0() { return 32 * (threadIdx.x >> 7); }
__device__ __forceinline__ int blk_c0() { return 32 * ((threadIdx.x >> 6) & 1); }
// row and column in the tile of element e of accumulator (bi, bj) of this lane
__device__ __forceinline__ int blk_row(int bi, int e) { return blk_r0() + 16 * bi + 4 * e + ((threadIdx.x & 63) >> 4); }
__device__ __forceinline__ int blk_col(int bj) { return blk_c0() + 16 * bj + (threadIdx.x & 15); }

__device__ __forceinline__ void blk_zero(Blk &b) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) b.c[bi][bj] = f64x4_t{0.0, 0.0, 0.0, 0.0};
}

__device__ __forceinline__ void blk_load(Blk &b, const double (*T)[kLd]) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 4; ++e) b.c[bi][bj][e] = T[blk_row(bi, e)][blk_col(bj)];
}

__device__ __forceinline__ void blk_store(double (*T)[kLd], const Blk &b) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 4; ++e) T[blk_row(bi, e)][blk_col(bj)] = b.c[bi][bj][e];
}

// b += s A^T B over the first K rows of A and B: C[r][c] += s sum_t A[t][r] B[t][c]
// (s = +1 or -1, applied to A's values exactly).
template <int K>
__device__ __forceinline__ void blk_atb(Blk &b, const double (*A)[kLd], const double (*B)[kLd], double s) {
  const int l = threadIdx.x & 63, r0 = blk_r0(), c0 = blk_c0();
#pragma unroll 4
  for (int t = 0; t < K; t += 4) {
    const int tr = t + (l >> 4);
    double a[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = s * A[tr][r0 + 16 * i + (l & 15)];
#pragma unroll
    for (int j = 0; j < 2; ++j) bv[j] = B[tr][c0 + 16 * j + (l & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) b.c[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], b.c[i][j], 0, 0, 0);
  }
}

// b += s A B: C[r][c] += s sum_t A[r][t] B[t][c], t < 64.
__device__ __forceinline__ void blk_ab(Blk &b, const double (*A)[kLd], const double (*B)[kLd], double s) {
  const int l = threadIdx.x & 63, r0 = blk_r0(), c0 = blk_c0();
#pragma unroll 4
  for (int t = 0; t < kNb; t += 4) {
    const int tc = t + (l >> 4);
    double a[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = s * A[r0 + 16 * i + (l & 15)][tc];
#pragma unroll
    for (int j = 0; j < 2; ++j) bv[j] = B[tc][c0 + 16 * j + (l & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) b.c[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], b.c[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// 1/sqrt(p) for p > 0: the hardware estimate, then two Newton steps for
// f(y) = 1/y^2 - p, y <- y (3 - p y^2) / 2, each of which about doubles the
// number of correct bits.
__device__ __forceinline__ double rsqrt_f64(double p) {
  double y = __builtin_amdgcn_rsq(p);
  const double h = 0.5 * p;
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(y, fma(-h * y, y, 0.5), y);
  return y;
}

// The diagonal 64 x 64 tile is worked on by the four wavefronts of the
// workgroup (256 threads), wavefront q holding rows 16q .. 16q+15 in
// registers, lane c column c; both routines below go block row by block row
// (16 rows), with one barrier per block row rather than one per row.
constexpr int kTileRows = kNb / (kCB / 64);  // rows per wavefront

// Cholesky (upper) of the tile S, right-looking by 16-row blocks.  Block jb
// is factored by its own wavefront alone: at step j it takes the pivot from
// lane j, scales row j by 1/R_jj (kept in rdiag for the inverse) and takes
// row j away from its later rows, reading R[j][i] from lane i of row j's
// register; no other wavefront is involved, so no barrier.  It then writes
// the block's rows to S (zero left of the diagonal) and, after a barrier,
// every wavefront with later rows subtracts the block's rank-16 product
// R_b^T R_b from them, reading R_b from LDS.  Only upper entries are ever
// read across lanes, so whatever the lower part of a row in registers turns
// into stays put.  Each row takes its pivots' updates in pivot order, as in
// the unblocked elimination.
__device__ __forceinline__ void chol_tile(double (*S)[kLd], const double *diag0, double *rdiag, int *bad) {
  constexpr int kR = kTileRows;
  const int c = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  double reg[kR];
#pragma unroll
  for (int m = 0; m < kR; ++m) reg[m] = S[kR * q + m][c];  // each wavefront reads and writes only its rows
  int badj = 0;
#pragma unroll 1
  for (int jb = 0; jb < kNb / kR; ++jb) {
    if (q == jb) {
#pragma unroll
      for (int jj = 0; jj < kR; ++jj) {
        const int j = jb * kR + jj;
        double p = readlane_f64(reg[jj], j);
        if (!(p > 1e-12 * diag0[j])) {
          badj = 1;
          p = 1.0;
        }
        const double y = rsqrt_f64(p);
        if (c == j)
          reg[jj] = p * y;
        else if (c > j)
          reg[jj] = reg[jj] * y;
        if (c == 0) rdiag[j] = y;
#pragma unroll
        for (int m = jj + 1; m < kR; ++m) reg[m] = fma(-readlane_f64(reg[jj], jb * kR + m), reg[jj], reg[m]);
      }
#pragma unroll
      for (int m = 0; m < kR; ++m) S[kR * jb + m][c] = kR * jb + m <= c ? reg[m] : 0.0;
    }
    __syncthreads();
    if (q > jb) {
#pragma unroll
      for (int t = 0; t < kR; ++t) {
        const double rc = S[kR * jb + t][c];
#pragma unroll
        for (int m = 0; m < kR; ++m) reg[m] = fma(-S[kR * jb + t][kR * q + m], rc, reg[m]);
      }
    }
  }
  if (c == 0 && badj) *bad = 1;
}

// X = U^-1 for the upper triangular tile U (LDS, zero below its diagonal;
// rdiag[j] = 1/U[j][j]), by back substitution in 16-row blocks from the
// last.  Rows of X start as the identity.  Block jb's wavefront finishes its
// rows alone: at step j (from the block's last row up) row j has had every
// term with a later index taken away, so scaling it by 1/U[j][j] makes it
// final, and the block's earlier rows take U[i][j] times it away (all in
// the wavefront's own lanes: column c of X stays in lane c).  It writes its
// rows to X and, after a barrier, every wavefront with earlier rows
// subtracts U[rows, block] X[block] from them.  Rows of X below the
// diagonal stay zero.
__device__ __forceinline__ void tri_inverse(const double (*U)[kLd], const double *rdiag, double (*X)[kLd]) {
  constexpr int kR = kTileRows;
  const int c = threadIdx.x & 63, q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  double x[kR];
#pragma unroll
  for (int m = 0; m < kR; ++m) x[m] = kR * q + m == c ? 1.0 : 0.0;
#pragma unroll 1
  for (int jb = kNb / kR - 1; jb >= 0; --jb) {
    if (q == jb) {
#pragma unroll
      for (int jj = kR - 1; jj >= 0; --jj) {
        const int j = jb * kR + jj;
        x[jj] = x[jj] * rdiag[j];
#pragma unroll
        for (int m = 0; m < jj; ++m) x[m] = fma(-U[kR * jb + m][j], x[jj], x[m]);
      }
#pragma unroll
      for (int m = 0; m < kR; ++m) X[kR * jb + m][c] = x[m];
    }
    __syncthreads();
    if (q < jb) {
#pragma unroll
      for (int t = 0; t < kR; ++t) {
        const double xc = X[kR * jb + t][c];
#pragma unroll
        for (int m = 0; m < kR; ++m) x[m] = fma(-U[kR * q + m][kR * jb + t], xc, x[m]);
      }
    }
  }
}

// R (upper, [k][k]) with G = R^T R, by the left-looking blocked Cholesky
// (64 x 64 blocks), one block row J at a time:
//     the diagonal block (diag_block, one workgroup; chol_tile, then the
//     block's inverse):
//         S = G_JJ - sum_{I<J} R_IJ^T R_IJ,   R_JJ = chol(S)      (in LDS)
//     the panel (chol_panel_kernel, one workgroup per block L > J):
//         R_JL = R_JJ^-T (G_JL - sum_{I<J} R_IJ^T R_IL)
// Block 0's diagonal is a launch of its own (chol_diag_kernel); every later
// diagonal block is factored by the panel launch before it, in the
// workgroup that writes the last block it needs, so a block row is one launch.
// The inverse of each diagonal block goes to Dinv[J] (64 x 64, upper): the
// panel and the solve for Q = Y R^-1 need only those.  A pivot that keeps
// at most 1e-12 of its column's squared norm (G_jj) means the block is
// numerically rank deficient (the fp32 products leave ~1e-14 there):
// status <- 1.
// LDS of one diagonal block's factorisation.
struct DiagLds {
  double diag0[kNb];
  double rdiag[kNb];
  int bad;
};

// Block row J's diagonal block: S = G_JJ - sum_{I<J} R_IJ^T R_IJ, R_JJ =
// chol(S), Dinv[J] = R_JJ^-1 (one workgroup; S, Di, Ta: 64 x 64 LDS tiles).
__device__ __forceinline__ void diag_block(const double *G, double *R, double *Dinv, int k, int J, uint32_t *status,
                           double (*S)[kLd], double (*Di)[kLd], double (*Ta)[kLd], DiagLds &D) {
  double *diag0 = D.diag0;
  int &s_bad = D.bad;
  const int tid = threadIdx.x;
  const int c0 = J * kNb, nJ = min(kNb, k - c0);
  if (tid == 0) s_bad = 0;
  load_tile(S, G, k, c0, c0, nJ, nJ);
  __syncthreads();
  if (tid < kNb) diag0[tid] = S[tid][tid];
  Blk acc;
  blk_load(acc, S);
  for (int I = 0; I < J; ++I) {
    __syncthreads();
    load_tile(Ta, R, k, I * kNb, c0, kNb, nJ);
    __syncthreads();
    blk_atb<kNb>(acc, Ta, Ta, -1.0);
  }
  __syncthreads();
  blk_store(S, acc);
  __syncthreads();
  // a partial block is padded with the identity, so that its factor is
  // chol(S) beside an identity block and every step below is uniform
  for (int e = tid; e < kNb * kNb; e += kCB) {
    const int r = e / kNb, c = e % kNb;
    if (r >= nJ || c >= nJ) S[r][c] = (r == c) ? 1.0 : 0.0;
  }
  if (tid < kNb && tid >= nJ) diag0[tid] = 1.0;
  __syncthreads();
  chol_tile(S, diag0, D.rdiag, &s_bad);
  __syncthreads();
  tri_inverse(S, D.rdiag, Di);
  __syncthreads();
  // R_JJ and Dinv[J] out (padding rows/columns of a partial block excluded)
  for (int e = tid; e < kNb * kNb; e += kCB) {
    const int r = e / kNb, c = e % kNb;
    if (r < nJ && c < nJ) R[(size_t)(c0 + r) * k + c0 + c] = S[r][c];
    Dinv[(size_t)J * kNb * kNb + e] = (r < nJ && c < nJ) ? Di[r][c] : 0.0;
  }
  if (tid == 0 && s_bad) *status = 1u;
}

__global__ void __launch_bounds__(kCB) chol_diag_kernel(const double *G, double *R, double *Dinv, int k, int J,
                                                        uint32_t *status) {
  __shared__ double S[kNb][kLd], Di[kNb][kLd], Ta[kNb][kLd];
  __shared__ DiagLds D;
  diag_block(G, R, Dinv, k, J, status, S, Di, Ta, D);
}

__global__ void __launch_bounds__(kCB) chol_panel_kernel(const double *G, double *R, double *Dinv, int k, int J,
                                                         uint32_t *status) {
  __shared__ double S[kNb][kLd], Di[kNb][kLd], Ta[kNb][kLd], Tb[kNb][kLd];
  __shared__ DiagLds D;
  const int c0 = J * kNb, nJ = min(kNb, k - c0);
  const int L = J + 1 + blockIdx.x;
  const int l0 = L * kNb, nL = min(kNb, k - l0);
  load_tiles2(S, G, k, c0, l0, nJ, nL, Di, Dinv + (size_t)J * kNb * kNb, kNb, 0, 0, kNb, kNb);
  __syncthreads();
  Blk acc;
  blk_load(acc, S);
  for (int I = 0; I < J; ++I) {
    __syncthreads();
    load_tiles2(Ta, R, k, I * kNb, c0, kNb, nJ, Tb, R, k, I * kNb, l0, kNb, nL);
    __syncthreads();
    blk_atb<kNb>(acc, Ta, Tb, -1.0);
  }
  __syncthreads();
  blk_store(S, acc);
  __syncthreads();
  // R_JL = Di^T S: out[r][c] = sum_{i <= r} Di[i][r] S[i][c]
  Blk out;
  blk_zero(out);
  blk_atb<kNb>(out, Di, S, 1.0);
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = blk_row(bi, e), c = blk_col(bj);
        if (r < nJ && c < nL) R[(size_t)(c0 + r) * k + l0 + c] = out.c[bi][bj][e];
      }
  // Block J+1's diagonal needs R_{I,J+1} for I <= J only, of which R_{J,J+1}
  // is the block this workgroup has just written: the workgroup of L = J+1
  // factors it here, which saves a launch per block row.
  if (blockIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // R_{J,J+1} is read back below
    __syncthreads();
    diag_block(G, R, Dinv, k, J + 1, status, S, Di, Ta, D);
  }
}

// Q = Y R^-1 ([d][k]) by a blocked forward substitution over the block
// columns: Q_J = (Y_J - sum_{I<J} Q_I R_IJ) R_JJ^-1.  Rows are independent:
// one workgroup per 64 rows, which reads back the Q blocks it wrote.
__global__ void __launch_bounds__(kCB) trsm_kernel(const double *Y, const double *R, const double *Dinv,
                                                   double *Q, int d, int k) {
  __shared__ double Ta[kNb][kLd], Tb[kNb][kLd];
  const int r0 = blockIdx.x * kNb, nr = min(kNb, d - r0);
  const int nbk = (k + kNb - 1) / kNb;
  for (int J = 0; J < nbk; ++J) {
    const int c0 = J * kNb, nJ = min(kNb, k - c0);
    __syncthreads();
    load_tile(Ta, Y, k, r0, c0, nr, nJ);
    __syncthreads();
    Blk acc;
    blk_load(acc, Ta);
    for (int I = 0; I < J; ++I) {
      __syncthreads();
      load_tiles2(Ta, Q, k, r0, I * kNb, nr, kNb, Tb, R, k, I * kNb, c0, kNb, nJ);
      __syncthreads();
      blk_ab(acc, Ta, Tb, -1.0);
    }
    __syncthreads();
    blk_store(Ta, acc);
    load_tile(Tb, Dinv + (size_t)J * kNb * kNb, kNb, 0, 0, kNb, kNb);
    __syncthreads();
    Blk out;
    blk_zero(out);
    blk_ab(out, Ta, Tb, 1.0);
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = blk_row(bi, e), c = blk_col(bj);
          if (r < nr && c < nJ) Q[(size_t)(r0 + r) * k + c0 + c] = out.c[bi][bj][e];
        }
    // this block column of Q is read back for the next ones
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// Split partials of G = Y^T Y (fp64, [d][k]): workgroup (tile, range) sums
// the 64 x 64 upper-triangle tile `tile` (bi <= bj) over rows
// [range * chunk, (range + 1) * chunk) of Y into P[range].
__global__ void __launch_bounds__(kCB) gram_split_kernel(const double *__restrict__ Y, double *__restrict__ P,
                                                         int d, int k, int chunk) {
  constexpr int KC = 32;
  __shared__ double Xs[KC][64 + 1];
  __shared__ double Ys[KC][64 + 1];
  const int t = (k + 63) / 64;
  int b = blockIdx.x, bi = 0;
  while (b >= t - bi) {
    b -= t - bi;
    ++bi;
  }
  const int i0 = bi * 64, j0 = (bi + b) * 64;
  const int r0 = blockIdx.y * chunk, r1 = min(d, r0 + chunk);
  const int tid = threadIdx.x;
  Blk acc;
  blk_zero(acc);
  // the next slab of rows is loaded into registers while this one is
  // multiplied (KC * 64 / kCB elements of each tile per thread)
  constexpr int PL = KC * 64 / kCB;
  double px[PL], py[PL];
  auto load = [&](int t0) {
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int e = tid + q * kCB, r = e / 64, c = e % 64;
      const bool ok = t0 + r < r1;
      px[q] = (ok && i0 + c < k) ? Y[(size_t)(t0 + r) * k + i0 + c] : 0.0;
      py[q] = (ok && j0 + c < k) ? Y[(size_t)(t0 + r) * k + j0 + c] : 0.0;
    }
  };
  if (r0 < r1) load(r0);
  for (int t0 = r0; t0 < r1; t0 += KC) {
    __syncthreads();  // the previous slab's products are done
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int e = tid + q * kCB;
      Xs[e / 64][e % 64] = px[q];
      Ys[e / 64][e % 64] = py[q];
    }
    __syncthreads();
    if (t0 + KC < r1) load(t0 + KC);
    blk_atb<KC>(acc, Xs, Ys, 1.0);
  }
  double *Pr = P + (size_t)blockIdx.y * k * k;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + blk_row(bi, e), j = j0 + blk_col(bj);
        if (i < k && j < k) Pr[(size_t)i * k + j] = acc.c[bi][bj][e];
      }
}

// G = sum of the S partials in range order, on the upper-triangle tiles
// (the only part of G the factorisation reads).
__global__ void __launch_bounds__(kCB) gram_reduce_kernel(const double *__restrict__ P, double *__restrict__ G,
                                                          int k, int S) {
  const size_t kk = (size_t)k * k;
  for (size_t e = (size_t)blockIdx.x * kCB + threadIdx.x; e < kk; e += (size_t)gridDim.x * kCB) {
    const int i = (int)(e / k), j = (int)(e % k);
    if (i / 64 > j / 64) continue;
    double s = 0.0;
    for (int r = 0; r < S; ++r) s += P[(size_t)r * kk + e];
    G[e] = s;
  }
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
void cholqr_pass(const double *Y, double *Q, double *G, double *R, double *Dinv, double *P, int d, int k,
                 uint32_t *status, hipStream_t s) {
  // G = Y^T Y: split partials, then their sum
  const int S = calib_gram_splits(d, k);
  const int chunk = (d + S - 1) / S;
  const int t = (k + 63) / 64;
  hipLaunchKernelGGL(gram_split_kernel, dim3(t * (t + 1) / 2, S), dim3(kCB), 0, s, Y, P, d, k, chunk);
  int rb = (int)(((size_t)k * k + kCB - 1) / kCB);
  if (rb > 2048) rb = 2048;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(rb), dim3(kCB), 0, s, P, G, k, S);
  const int nbk = (k + kNb - 1) / kNb;
  hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(kCB), 0, s, G, R, Dinv, k, 0, status);
  for (int J = 0; J + 1 < nbk; ++J)  // block row J's panel, then block J+1's diagonal
    hipLaunchKernelGGL(chol_panel_kernel, dim3(nbk - J - 1), dim3(kCB), 0, s, G, R, Dinv, k, J, status);
  hipLaunchKernelGGL(trsm_kernel, dim3((d + kNb - 1) / kNb), dim3(kCB), 0, s, Y, R, Dinv, Q, d, k);
}

// C = sum of the `splits` fp32 partials [splits][count] (part stride count),
// as three bf16 parts (part stride count).
__global__ void __launch_bounds__(kCB) zsum_split_kernel(const float *__restrict__ part, int splits,
                                                         uint16_t *__restrict__ C, size_t count) {
  const size_t e = (size_t)blockIdx.x * kCB + threadIdx.x;
  if (e >= count) return;
  float v = part[e];
  for (int z = 1; z < splits; ++z) v += part[(size_t)z * count + e];
  uint16_t pt[3];
  split3(v, pt);
  C[e] = pt[0];
  C[count + e] = pt[1];
  C[2 * count + e] = pt[2];
}

// One sweep's products on the matrix cores: Z^T = V^T A^T (as three bf16
// parts), then Y = A^T Z (fp64).  Z^T has k x n outputs over K = d: with
// one workgroup per 64 x 64 tile that is about one workgroup per CU, whose
// LDS writes, barrier, LDS reads and matrix products follow one another
// with nothing to fill the gaps, so K is split (up to four ways, to two
// workgroups per CU) where the fp32 partials fit in y2, which is not in use
// until the factorisation; a small kernel adds them and splits the sum into
// parts.
void mfma_products(const CalibArgs &c, hipStream_t s) {
  MGemm g1{};
  g1.P = c.vt3;
  g1.Q = static_cast<const uint16_t *>(c.A);
  g1.C = c.zt3;
  g1.zero = static_cast<const u32x4_t *>(c.zeros);
  g1.M = c.k;
  g1.N = c.n;
  g1.K = c.d;
  g1.ldp = c.dp;
  g1.ldq = c.d;
  g1.ldc = c.np;
  g1.sp = (size_t)c.k * c.dp;
  g1.sc = (size_t)c.k * c.np;
  // K splits: 1, 2 or 4, as many as bring the grid to two workgroups per
  // CU, fewer where the partials would not fit in y2
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t tiles = (int64_t)((c.k + 63) / 64) * (c.np / 64);
  int splits = 1;
  while (splits < 4 && tiles * splits < 2 * cus) splits *= 2;
  while (splits > 1 && (uint64_t)splits * c.k * c.np * sizeof(float) > (uint64_t)c.d * c.k * sizeof(double))
    splits /= 2;
  if (c.d < 1024) splits = 1;
  if (splits > 1) {
    g1.C = c.y2;
    hipLaunchKernelGGL((mgemm_kernel<3, 1, 2, 1>), dim3((c.k + 63) / 64, c.np / 64, splits), dim3(kCB), 0, s, g1);
    const size_t count = (size_t)c.k * c.np;
    hipLaunchKernelGGL(zsum_split_kernel, dim3((unsigned)((count + kCB - 1) / kCB)), dim3(kCB), 0, s,
                       static_cast<const float *>(static_cast<void *>(c.y2)), splits, c.zt3, count);
  } else {
    hipLaunchKernelGGL((mgemm_kernel<3, 1, 0, 1>), dim3((c.k + 63) / 64, c.np / 64), dim3(kCB), 0, s, g1);
  }
  MGemm g2{};
  g2.P = c.at;
  g2.Q = c.zt3;
  g2.C = c.y;
  g2.zero = g1.zero;
  g2.M = c.d;
  g2.N = c.k;
  g2.K = c.np;
  g2.ldp = c.np;
  g2.ldq = c.np;
  g2.ldc = c.k;
  g2.sq = (size_t)c.k * c.np;
  hipLaunchKernelGGL((mgemm_kernel<1, 3, 1, 3>), dim3((c.d + 63) / 64, (c.k + 63) / 64), dim3(kCB), 0, s, g2);
}

template <typename TY>
void split_t(const TY *Y, const CalibArgs &c, hipStream_t s) {
  hipLaunchKernelGGL((split_t_kernel<TY>), dim3(c.dp / 64, (c.k + 63) / 64), dim3(kCB), 0, s, Y, c.vt3, c.d, c.k,
                     c.dp);
}

template <typename T>
hipError_t run(const CalibArgs &c, hipStream_t s) {
  const T *A = static_cast<const T *>(c.A);
  if (c.mfma) {
    hipLaunchKernelGGL(transpose_pad_kernel, dim3(c.np / 64, (c.d + 63) / 64), dim3(kCB), 0, s,
                       reinterpret_cast<const uint16_t *>(A), c.at,
                       static_cast<uint32_t *>(const_cast<void *>(c.zeros)), c.n, c.d, c.np);
    split_t(static_cast<const T *>(c.V0), c, s);
  } else {
    convert(static_cast<const T *>(c.V0), c.vw, (size_t)c.d * c.k, s);
  }
  for (int it = 0; it < c.iters; ++it) {
    if (c.mfma) {
      mfma_products(c, s);
    } else {
      gemm<T, float, float, float, false>(A, c.vw, c.z, c.n, c.k, c.d, s);    // Z = A V      [n][k]
      gemm<T, float, double, float, true>(A, c.z, c.y, c.d, c.k, c.n, s);     // Y = A^T Z    [d][k]
    }
    cholqr_pass(c.y, c.y2, c.g, c.r, c.dinv, c.gpart, c.d, c.k, c.status, s);  // y2 = Q(y)
    cholqr_pass(c.y2, c.y, c.g, c.r, c.dinv, c.gpart, c.d, c.k, c.status, s);  // y = Q(y2): orthogonal to rounding
    if (it + 1 < c.iters) {
      if (c.mfma)
        split_t(c.y, c, s);
      else
        convert(c.y, c.vw, (size_t)c.d * c.k, s);
    }
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
