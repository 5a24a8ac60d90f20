// Batched gated map (many tokens through one bf16 map) on gfx950 MFMA.
//
// Method: "Gated Subspace Inference for Transformer Acceleration"
// (S. J. Thomas, 2026), technical summary (GSI-TS) §2.1-§2.2, applied to a
// batch: every token gets its own gate, fast tokens are computed together as
// Y_f = G_f M^T and slow tokens as Y_s = X_s W^T, so M and W are each read
// once per launch however many tokens take the path.
//
//   bproj_kernel : split-K GEMM G = X V_k with v_mfma_f32_16x16x32_bf16 and the
//                  per-token ||x||^2; a V_k chunk is staged in LDS transposed
//                  ([col][k]) so each lane reads its 8-element K slice as one
//                  16-byte LDS read.  Partials [S][T][k] fp32.
//   bgate_kernel : one workgroup per token: sums the S partials in a fixed
//                  order, forms ||g||^2, rho and the gate, writes g as bf16
//                  hi + lo (g = hi + lo to ~2^-16) for the fast GEMM.
//   bout_kernel  : one launch per path.  Each workgroup compacts the tokens
//                  of its path (deterministic order), takes 64 output columns
//                  and all those tokens (256 per pass) and runs
//                  v_mfma_f32_32x32x16_bf16 over K chunks of 64 with a
//                  register-staged prefetch pipeline (see below).
//
// MFMA operand layouts (checked on the device): for 32x32x16, lane l holds
// A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32], e = 0..7, and
// accumulator i of lane l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]; for
// 16x16x32, A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16] and
// C[4 (l / 16) + i][l % 16].
#include <hip/hip_runtime.h>

#include <cfloat>

#include "gsi_internal.h"

namespace gsi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16-byte piece as a native vector (HIP's uint4 is a struct whose copies
// become memcpys that keep staged values in scratch memory).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float rho_of(float xx, float gg) {
  if (!(xx <= FLT_MAX) || !(gg <= FLT_MAX)) return __builtin_nanf("");
  if (xx == 0.f) return 0.f;
  const float t = 1.f - gg / xx;
  return t > 0.f ? sqrtf(t) : 0.f;
}

}  // namespace

// ---------------------------------------------------------------------------
// G partials: tile of 64 tokens x 64 columns of g over the rows [i0, i1) of V_k.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) bproj_kernel(BArgs a) {
  __shared__ __align__(16) uint16_t Vt[64][kBatchKc + 8];  // V chunk transposed: [col][row]
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * 64;
  const int j0 = blockIdx.y * 64;
  const int s = blockIdx.z;
  const int i0 = s * a.kc;
  const int rows = min(a.kc, a.d - i0);
  const uint16_t *V = static_cast<const uint16_t *>(a.V);
  const uint16_t *X = static_cast<const uint16_t *>(a.x);

  // stage V[i0 + r][j0 + c] as Vt[c][r] (zero outside the map)
  for (int v = tid; v < kBatchKc * 8; v += kBlock) {
    const int r = v >> 3, cg = v & 7;
    const int j = j0 + cg * 8;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && j < a.k) u = *reinterpret_cast<const uint4 *>(V + (size_t)(i0 + r) * a.k + j);
    const uint16_t *h = reinterpret_cast<const uint16_t *>(&u);
#pragma unroll
    for (int e = 0; e < 8; ++e) Vt[cg * 8 + e][r] = h[e];
  }
  __syncthreads();

  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int tok = t0 + wave * 16 + (lane & 15);
  const bool tok_ok = tok < a.n;
  const int kq = 8 * (lane >> 4);
  float xx = 0.f;
  for (int kk = 0; kk < rows; kk += 32) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (tok_ok && kk + kq < rows) u = *reinterpret_cast<const uint4 *>(X + (size_t)tok * a.d + i0 + kk + kq);
    if (blockIdx.y == 0) {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(&u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = bf2f(h[e]);
        xx = fmaf(f, f, xx);
      }
    }
    const bf16x8_t A = as_bf16x8(u);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 b = *reinterpret_cast<const uint4 *>(&Vt[c * 16 + (lane & 15)][kk + kq]);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(b), acc[c], 0, 0, 0);
    }
  }
  float *P = a.part + (size_t)s * a.n * a.k;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + wave * 16 + 4 * (lane >> 4) + i;
      const int j = j0 + c * 16 + (lane & 15);
      if (t < a.n && j < a.k) P[(size_t)t * a.k + j] = acc[c][i];
    }
  }
  if (blockIdx.y == 0) {
    // the four lanes holding one token's K slices: lane, lane^16, lane^32, lane^48
    xx += __shfl_xor(xx, 16, 64);
    xx += __shfl_xor(xx, 32, 64);
    if (lane < 16 && tok_ok) a.xxp[(size_t)s * a.n + tok] = xx;
  }
}

// ---------------------------------------------------------------------------
// Gate per token: one workgroup per token; every split partial of a column
// is requested before any is summed (fixed order), so a token costs one or
// two memory round trips.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(kBlock) bgate_kernel(BArgs a) {
  __shared__ float sh[kWaves];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  float gg = 0.f;
  for (int j = tid; j < a.kpad; j += kBlock) {
    float g = 0.f;
    if (j < a.k) {
      const float *p = a.part + (size_t)t * a.k + j;
      const size_t stride = (size_t)a.n * a.k;
      int s = 0;
      for (; s + 16 <= a.splits; s += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = p[(size_t)(s + i) * stride];
#pragma unroll
        for (int i = 0; i < 16; ++i) g += v[i];
      }
      for (; s < a.splits; ++s) g += p[(size_t)s * stride];
    }
    gg = fmaf(g, g, gg);
    const uint16_t hi = f2bf(g);
    const uint16_t lo = f2bf(g - bf2f(hi));
    a.ghi[(size_t)t * a.kpad + j] = hi;
    a.glo[(size_t)t * a.kpad + j] = lo;
  }
  float xp = 0.f;
  for (int s = tid; s < a.splits; s += kBlock) xp += a.xxp[(size_t)s * a.n + t];
  // workgroup sums in a fixed order
  gg = wsum(gg);
  xp = wsum(xp);
  if ((tid & 63) == 0) sh[tid >> 6] = gg;
  __syncthreads();
  float ggt = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) ggt += sh[i];
  __syncthreads();
  if ((tid & 63) == 0) sh[tid >> 6] = xp;
  __syncthreads();
  float xx = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) xx += sh[i];
  if (tid == 0) {
    const float rho = rho_of(xx, ggt);
    const int slow = MODE == 2 ? 1 : (MODE == 1 ? 0 : !(rho < a.eps));
    a.flags[t] = slow;
    if (a.rho) a.rho[t] = rho;
    if (a.slow) a.slow[t] = (uint8_t)slow;
  }
}

// ---------------------------------------------------------------------------
// Outputs: 64 columns x all tokens of one path per workgroup.
//
// PATH 0 (fast): A = G as bf16 hi + lo [n][kpad], B = the image tile (M's
// 64-row tile is already in MFMA order); PATH 1 (slow): A = X [n][d], B = 64
// rows of W.  Each wavefront owns 64 tokens (two 32-row MFMA tiles) x 64
// columns.  K advances in chunks of 64: every thread prefetches its share of
// the B chunk and every wavefront its own token rows of the A chunk two
// chunks ahead into registers; the B chunk goes through a double-buffered
// LDS tile shared by the four wavefronts.  One workgroup per CU streams its
// 64 rows of W (or M) exactly once per 256 tokens.
// ---------------------------------------------------------------------------
template <int PATH>
struct OutStage {
  static constexpr int NA = PATH == 0 ? 2 : 1;  // A matrices: (hi, lo) or (x)
  u32x4_t b0, b1;                               // this thread's two 16-byte pieces of B
  u32x4_t a[NA][2][4];                          // [matrix][m subtile][k step]
};

// Address of the 16-byte piece v (0..511) of the B chunk at K offset kk0.
template <int PATH>
__device__ __forceinline__ const u32x4_t *out_b_ptr(const BArgs &a, int kk0, int o0, int v,
                                                    const u32x4_t *zero) {
  if (PATH == 0) {
    const int cg = v >> 6, r = v & 63;
    const int kg = kk0 + cg * 8;
    const u32x4_t *p =
        static_cast<const u32x4_t *>(a.M) + ((size_t)(o0 / 64) * (a.k / 8) + kg / 8) * 64 + r;
    return kg < a.k ? p : zero;
  }
  const int r = v >> 3, cg = v & 7;
  const int kg = kk0 + cg * 8;
  const u32x4_t *p =
      reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.W) + (size_t)(o0 + r) * a.d + kg);
  return (o0 + r < a.d_out && kg < a.d) ? p : zero;
}

// Loads are never predicated and never followed by a select on the data: an
// out-of-range piece is read from a 256-byte zero block of the workspace
// instead (the select is on the address), so the compiler can keep every
// prefetched load in flight.
template <int PATH>
__device__ __forceinline__ void out_load(OutStage<PATH> &st, const BArgs &a, int kk0, int o0,
                                         const int (&tokr)[2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const u32x4_t *zero = static_cast<const u32x4_t *>(a.zeros);
  st.b0 = *out_b_ptr<PATH>(a, kk0, o0, tid, zero);
  st.b1 = *out_b_ptr<PATH>(a, kk0, o0, tid + kBlock, zero);
  const int K = PATH == 0 ? a.kpad : a.d;
  const int kq = 8 * (lane >> 5);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kg = kk0 + ks * 16 + kq;
      const bool ok = tokr[m] >= 0 && kg < K;
      if (PATH == 0) {
        const size_t off = (size_t)tokr[m] * a.kpad + kg;
        st.a[0][m][ks] = *(ok ? reinterpret_cast<const u32x4_t *>(a.ghi + off) : zero);
        st.a[OutStage<PATH>::NA - 1][m][ks] = *(ok ? reinterpret_cast<const u32x4_t *>(a.glo + off) : zero);
      } else {
        const size_t off = (size_t)tokr[m] * a.d + kg;
        st.a[0][m][ks] =
            *(ok ? reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) + off) : zero);
      }
    }
}

template <int PATH>
__device__ __forceinline__ void out_store_b(const OutStage<PATH> &st, u32x4_t (*Bs)[64]) {
  const int tid = threadIdx.x;
  const int v1 = tid + kBlock;
  if (PATH == 0) {
    Bs[tid >> 6][tid & 63] = st.b0;
    Bs[v1 >> 6][v1 & 63] = st.b1;
  } else {
    Bs[tid & 7][tid >> 3] = st.b0;
    Bs[v1 & 7][v1 >> 3] = st.b1;
  }
}

template <int PATH>
__device__ __forceinline__ void out_mma(const OutStage<PATH> &st, const u32x4_t (*Bs)[64],
                                        f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8_t b0 = as_bf16x8(Bs[ks * 2 + (lane >> 5)][lane & 31]);
    const bf16x8_t b1 = as_bf16x8(Bs[ks * 2 + (lane >> 5)][32 + (lane & 31)]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < OutStage<PATH>::NA; ++q) {
        const bf16x8_t A = as_bf16x8(st.a[q][m][ks]);
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b0, acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b1, acc[m][1], 0, 0, 0);
      }
  }
}

template <int PATH>
__global__ void __launch_bounds__(kBlock, 1) bout_kernel(BArgs a) {
  __shared__ __align__(16) u32x4_t Bs[2][8][64];  // double-buffered 64-wide K chunk: [k group][column]
  __shared__ int16_t idx[kMaxBatch];
  __shared__ int scan[kBlock];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int o0 = blockIdx.x * 64;
  const int n = a.n;

  // tokens of this path in increasing order
  const int per = (n + kBlock - 1) / kBlock;
  const int c0 = tid * per;
  int mine = 0;
  for (int i = 0; i < per; ++i)
    if (c0 + i < n && a.flags[c0 + i] == PATH) ++mine;
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kBlock; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  {
    int w = scan[tid] - mine;
    for (int i = 0; i < per; ++i)
      if (c0 + i < n && a.flags[c0 + i] == PATH) idx[w++] = (int16_t)(c0 + i);
  }
  const int count = scan[kBlock - 1];
  __syncthreads();
  if (count == 0) return;

  const int K = PATH == 0 ? a.kpad : a.d;
  const int nch = (K + 63) / 64;
  uint16_t *Y = static_cast<uint16_t *>(a.y);

  for (int base = 0; base < count; base += 256) {
    int tokr[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int row = base + wave * 64 + m * 32 + (lane & 31);
      tokr[m] = row < count ? idx[row] : -1;
    }
    f32x16_t acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][c][i] = 0.f;

    // Three named stages (an array of stages would live in scratch memory):
    // chunk i is consumed while chunks i+1 and i+2 load.  The loop is
    // branch-free and runs a multiple of three chunks; chunks past K read the
    // zero block and wavefronts without tokens multiply zeros.
    OutStage<PATH> s0, s1, s2;
#define GSI_OUT_STEP(cur, ahead, i)                       \
  do {                                                    \
    out_load<PATH>(ahead, a, ((i) + 2) * 64, o0, tokr);   \
    out_store_b<PATH>(cur, Bs[(i) & 1]);                  \
    __syncthreads();                                      \
    out_mma<PATH>(cur, Bs[(i) & 1], acc);                 \
  } while (0)
    out_load<PATH>(s0, a, 0, o0, tokr);
    out_load<PATH>(s1, a, 64, o0, tokr);
    for (int i = 0; i < nch; i += 3) {
      GSI_OUT_STEP(s0, s2, i);
      GSI_OUT_STEP(s1, s0, i + 1);
      GSI_OUT_STEP(s2, s1, i + 2);
    }
#undef GSI_OUT_STEP
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = base + wave * 64 + m * 32 + 8 * (i / 4) + 4 * (lane >> 5) + (i & 3);
          const int col = o0 + c * 32 + (lane & 31);
          if (row < count && col < a.d_out) Y[(size_t)idx[row] * a.d_out + col] = f2bf(acc[m][c][i]);
        }
  }
}

// ---------------------------------------------------------------------------
// Image M = W V_k (bf16, once per map): workgroup = 64 rows of W x 64 columns
// of V_k over all of d.  V_k is staged 256 rows at a time, transposed in LDS;
// wavefront w multiplies rows 16 w.. of the W tile (v_mfma_f32_16x16x32_bf16).
// The result is rounded to bf16 into the tiled image layout.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock)
    bprep_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ V,
                 uint16_t *__restrict__ M, int d, int d_out, int k) {
  __shared__ __align__(16) uint16_t Vt[64][kBatchKc + 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int o0 = blockIdx.x * 64;
  const int j0 = blockIdx.y * 64;
  const int o = o0 + wave * 16 + (lane & 15);
  const bool row_ok = o < d_out;
  const int kq = 8 * (lane >> 4);
  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < d; i0 += kBatchKc) {
    const int rows = min(kBatchKc, d - i0);
    __syncthreads();
    for (int v = tid; v < kBatchKc * 8; v += kBlock) {
      const int r = v >> 3, cg = v & 7;
      const int j = j0 + cg * 8;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows && j < k) u = *reinterpret_cast<const uint4 *>(V + (size_t)(i0 + r) * k + j);
      const uint16_t *h = reinterpret_cast<const uint16_t *>(&u);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[cg * 8 + e][r] = h[e];
    }
    __syncthreads();
    for (int kk = 0; kk < rows; kk += 32) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok && kk + kq < rows) u = *reinterpret_cast<const uint4 *>(W + (size_t)o * d + i0 + kk + kq);
      const bf16x8_t A = as_bf16x8(u);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 b = *reinterpret_cast<const uint4 *>(&Vt[c * 16 + (lane & 15)][kk + kq]);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, as_bf16x8(b), acc[c], 0, 0, 0);
      }
    }
  }
  // tiled image: element (r, j) at ((r/64)(k/8) + j/8) 512 + (r%64) 8 + j%8
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = o0 + wave * 16 + 4 * (lane >> 4) + i;  // rows past d_out hold zeros (W rows read as 0)
      const int j = j0 + c * 16 + (lane & 15);
      if (j < k) M[((size_t)(r / 64) * (k / 8) + j / 8) * 512 + (r % 64) * 8 + (j % 8)] = f2bf(acc[c][i]);
    }
}

hipError_t launch_prepare_bf16(const void *W, const void *V, void *M, int d, int d_out, int k,
                               hipStream_t s) {
  hipLaunchKernelGGL(bprep_kernel, dim3((d_out + 63) / 64, (k + 63) / 64), dim3(kBlock), 0, s,
                     static_cast<const uint16_t *>(W), static_cast<const uint16_t *>(V),
                     static_cast<uint16_t *>(M), d, d_out, k);
  return hipGetLastError();
}

hipError_t launch_batched(const BArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(bproj_kernel, dim3((a.n + 63) / 64, (a.k + 63) / 64, a.splits), dim3(kBlock), 0,
                     s, a);
  const dim3 gg(a.n);
  if (a.mode == 1)
    hipLaunchKernelGGL(bgate_kernel<1>, gg, dim3(kBlock), 0, s, a);
  else if (a.mode == 2)
    hipLaunchKernelGGL(bgate_kernel<2>, gg, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(bgate_kernel<0>, gg, dim3(kBlock), 0, s, a);
  const dim3 go((a.d_out + 63) / 64);
  hipLaunchKernelGGL((bout_kernel<0>), go, dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL((bout_kernel<1>), go, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace gsi
