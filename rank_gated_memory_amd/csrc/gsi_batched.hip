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
//                  ([col][k], swizzled by column group) so each lane reads
//                  its 8-element K slice as one 16-byte LDS read.  Partials
//                  [S][T][k] fp32.
//   bgate_kernel : one workgroup per token: sums the S partials in a fixed
//                  order, forms ||g||^2, rho and the gate, writes g as bf16
//                  hi + lo (g = hi + lo to ~2^-16) for the fast GEMM.
//   bout_kernel  : every output of the call in one launch, one workgroup of
//                  eight wavefronts per CU.  Each workgroup compacts the
//                  tokens of each path from the gate flags itself
//                  (deterministic order).  A path with 1 to kThin tokens is
//                  a row stream: the matrix in blocks of 16 (fast) or 32
//                  (slow) rows, two blocks at a time (one per half of the
//                  workgroup), v_mfma_f32_16x16x32_bf16 (bthin_path).  A path
//                  with more: fast, items of 64 tokens x 256 output rows,
//                  the image read straight from its tiled layout in MFMA
//                  operand order and g's planes staged in LDS
//                  (wide_fast_item); slow, 64-column tiles, all of the
//                  path's tokens (256 per pass, eight wavefronts of 32)
//                  against the tile with v_mfma_f32_32x32x16_bf16 over K
//                  chunks of 64, register-staged prefetch, y leaving through
//                  LDS in 16-byte pieces (bout_path).
//   bprep_kernel : the image M = W V_k (once per map).
//
// MFMA operand layouts (checked on the device): for 32x32x16, lane l holds
// A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32], e = 0..7, and
// accumulator i of lane l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]; for
// 16x16x32, A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16] and
// C[4 (l / 16) + i][l % 16].
#include <hip/hip_runtime.h>

#include <cfloat>

#include "gsi_batched.h"
#include "gsi_gram.h"

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

// Keeps the compiler from moving LDS accesses across this point; the LDS
// accesses of one wavefront complete in order, so this suffices between a
// wavefront's writes to its own region and its reads of them.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float rho_of(float xx, float gg) {
  if (!(xx <= FLT_MAX) || !(gg <= FLT_MAX)) return __builtin_nanf("");
  if (xx == 0.f) return 0.f;
  const float t = 1.f - gg / xx;
  return t > 0.f ? sqrtf(t) : 0.f;
}

}  // namespace

namespace {

// Inclusive workgroup scan of two counters at once over the NT threads:
// within each wavefront by shuffles, then the wavefront totals through LDS
// (sh: NT / 64 entries), so the whole scan waits on one barrier.  Returns
// the thread's inclusive prefix; *tot receives the workgroup totals.
template <int NT>
__device__ __forceinline__ int2 block_scan2(int2 v, int2 *sh, int2 *tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ux = __shfl_up(v.x, off, 64), uy = __shfl_up(v.y, off, 64);
    if (lane >= off) {
      v.x += ux;
      v.y += uy;
    }
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int2 before = make_int2(0, 0), all = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int2 t = sh[w];
    if (w < wave) {
      before.x += t.x;
      before.y += t.y;
    }
    all.x += t.x;
    all.y += t.y;
  }
  *tot = all;
  return make_int2(v.x + before.x, v.y + before.y);
}

// Tokens of each path in increasing order, from the gate flags: the fast
// tokens in idx[0, nf), the slow ones in idx[nf, n).  Every output
// workgroup (NT threads) compacts the n flags itself (one load per thread at
// n = 256 and a two-counter scan; scan: NT / 64 entries), so the gate needs
// no grid-wide step.  Returns (nf, ns).
template <int NT>
__device__ __forceinline__ int2 path_lists(const BArgs &a, int16_t *idx, int2 *scan) {
  const int tid = threadIdx.x;
  const int per = (a.n + NT - 1) / NT;
  const int c0 = tid * per;
  constexpr int kPer = (kMaxBatch + NT - 1) / NT;
  int fl[kPer];
  int2 mine = make_int2(0, 0);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    fl[i] = (i < per && c0 + i < a.n) ? a.flags[c0 + i] : -1;
    mine.x += fl[i] == 0;
    mine.y += fl[i] == 1;
  }
  int2 tot;
  const int2 inc = block_scan2<NT>(mine, scan, &tot);
  int wf = inc.x - mine.x, ws = tot.x + inc.y - mine.y;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (fl[i] == 0) idx[wf++] = (int16_t)(c0 + i);
    if (fl[i] == 1) idx[ws++] = (int16_t)(c0 + i);
  }
  __syncthreads();
  return tot;
}

}  // namespace

// ---------------------------------------------------------------------------
// G partials: tile of 64 tokens x 64 columns of g over the rows [i0, i1) of
// V_k (v_mfma_f32_16x16x32_bf16, the V_k chunk transposed in LDS).  Every
// load of the tile is issued before the first is used (x fragments, then the
// V_k chunk), so the workgroup waits for memory about once.  Partials
// [splits][n][k] and ||x||^2 partials [splits][n] are summed by the gate
// kernel after the launch boundary.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kBlock) bproj_kernel(BArgs a) {
  constexpr int KS = kBatchKc / 32;                         // k-steps of 32 rows per split
  constexpr int VL = kBatchKc * 8 / kBlock;                 // 16-byte pieces of V per thread
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
  // one zero piece per lane: with a uniform fallback address the compiler
  // turns the address select into a branch around the load
  const u32x4_t *zero = static_cast<const u32x4_t *>(a.zeros) + (lane & 15);

  const int tok = t0 + wave * 16 + (lane & 15);
  const bool tok_ok = tok < a.n;
  const int kq = 8 * (lane >> 4);
  u32x4_t xv[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const int kk = q * 32 + kq;
    const bool ok = tok_ok && kk < rows;
    xv[q] = *(ok ? reinterpret_cast<const u32x4_t *>(X + (size_t)tok * a.d + i0 + kk) : zero);
  }
  u32x4_t vv[VL];
#pragma unroll
  for (int q = 0; q < VL; ++q) {
    const int v = tid + q * kBlock;
    const int r = v >> 3, j = j0 + (v & 7) * 8;
    const bool ok = r < rows && j < a.k;
    vv[q] = *(ok ? reinterpret_cast<const u32x4_t *>(V + (size_t)(i0 + r) * a.k + j) : zero);
  }
  // stage V[i0 + r][j0 + c] as Vt[c][r ^ 8 (c / 8)] (zero outside the map).
  // A wavefront's stores cover 8 rows x 8 column groups; the row pitch is a
  // multiple of 128 bytes, so unswizzled the eight column groups would share
  // banks.  XOR-ing r with 8 (c / 8) spreads them and keeps every aligned
  // group of 8 rows contiguous for the 16-byte operand reads.
#pragma unroll
  for (int q = 0; q < VL; ++q) {
    const int v = tid + q * kBlock;
    const int r = v >> 3, cg = v & 7;
    const int rs = r ^ (8 * cg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Vt[cg * 8 + 2 * e][rs] = (uint16_t)(vv[q][e] & 0xffffu);
      Vt[cg * 8 + 2 * e + 1][rs] = (uint16_t)(vv[q][e] >> 16);
    }
  }
  __syncthreads();

  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float xx = 0.f;
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    if (q * 32 >= rows) break;
    if (blockIdx.y == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(xv[q][e] << 16), hi = __uint_as_float(xv[q][e] & 0xffff0000u);
        xx = fmaf(lo, lo, xx);
        xx = fmaf(hi, hi, xx);
      }
    }
    const bf16x8_t A = as_bf16x8(xv[q]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = c * 16 + (lane & 15);
      const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&Vt[col][(q * 32 + kq) ^ (8 * (col >> 3))]);
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
// Gate per token: one workgroup per token sums the split partials of g in
// split order (every partial of a column requested before any is summed),
// writes g as bf16 hi + lo (g = hi + lo to ~2^-16) for the fast GEMM, and
// forms rho and the gate (GSI-TS §2.2).  The flags are all the output
// kernels need: each of their workgroups compacts the tokens itself.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(kBlock) bgate_kernel(BArgs a) {
  __shared__ float sh[kWaves];
  __shared__ float gl[1024];  // g of the token, for the exact rho
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
    if (a.G && j < a.k) gl[j] = g;
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
  float q = 0.f;
  if (a.G) q = gram_quadratic<2, kBlock>(a.G, a.k, gl, sh);
  if (tid == 0) {
    const float rho = a.G ? rho_exact(xx, ggt, q) : rho_of(xx, ggt);
    const int slow = MODE == 2 ? 1 : (MODE == 1 ? 0 : !(rho < a.eps));
    a.flags[t] = slow;
    if (a.rho) a.rho[t] = rho;
    if (a.slow) a.slow[t] = (uint8_t)slow;
  }
}

// ---------------------------------------------------------------------------
// Outputs: 64 columns x all tokens of one path per workgroup (bout_path; the
// launch uses it for the slow path, the fast path taking wide_fast_item).
//
// PATH 0 (fast): A = G as bf16 hi + lo [n][kpad], B = the image tile (M's
// 64-row tile is already in MFMA order); PATH 1 (slow): A = X [n][d], B = 64
// rows of W.  A workgroup has eight wavefronts, two per SIMD, so that one
// wavefront's products run while the other waits on its loads, its LDS
// traffic or the barrier; each owns 32 tokens (one 32-row MFMA tile) x 64
// columns, 256 tokens per round.  K advances in chunks of 64: every thread
// prefetches its 16-byte piece of the B chunk and every wavefront its own
// token rows of the A chunk D-1 chunks ahead into registers; the B chunk
// goes through a double-buffered LDS tile shared by the eight wavefronts.
// One workgroup per CU streams its 64 rows of W (or M) exactly once per 256
// tokens.  The A chunk is loaded row-contiguously (eight lanes per 128-byte
// token row) and transposed through the wavefront's own LDS region, since
// loading it in operand layout would touch a different token row, and cache
// line, in every lane.
// ---------------------------------------------------------------------------
#ifndef GSI_OUT_DEPTH_FAST
#define GSI_OUT_DEPTH_FAST 2
#endif
#ifndef GSI_OUT_DEPTH_SLOW
#define GSI_OUT_DEPTH_SLOW 2
#endif

constexpr int kOutWaves = 8;
constexpr int kOutThreads = kOutWaves * 64;
constexpr int kOutTok = 32;                     // tokens of a wavefront in a round
constexpr int kOutRound = kOutWaves * kOutTok;  // tokens of a round

template <int PATH>
struct OutStage {
  static constexpr int NA = PATH == 0 ? 2 : 1;  // A matrices: (hi, lo) or (x)
  static constexpr int kDepth = PATH == 0 ? GSI_OUT_DEPTH_FAST : GSI_OUT_DEPTH_SLOW;  // stages in the ring
  u32x4_t b;                                    // this thread's 16-byte piece of B
  u32x4_t a[NA][4];                             // piece i * 64 + lane of the 32 x 128-byte A chunk
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
                                         const int (&tk)[4], const u32x4_t *zero) {
  const int tid = threadIdx.x, lane = tid & 63;
  st.b = *out_b_ptr<PATH>(a, kk0, o0, tid, zero);
  const int K = PATH == 0 ? a.k : a.d;
  const int kg = kk0 + (lane & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = tk[i] >= 0 && kg < K;
    if (PATH == 0) {
      const size_t off = (size_t)tk[i] * a.kpad + kg;
      st.a[0][i] = *(ok ? reinterpret_cast<const u32x4_t *>(a.ghi + off) : zero);
      st.a[OutStage<PATH>::NA - 1][i] = *(ok ? reinterpret_cast<const u32x4_t *>(a.glo + off) : zero);
    } else {
      const size_t off = (size_t)tk[i] * a.d + kg;
      st.a[0][i] =
          *(ok ? reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) + off) : zero);
    }
  }
}

// Column slot of piece (k group cg, column c) in the B chunk.  The slow
// path's eight lanes of one W row write the eight k groups of one column,
// 1 KiB apart in [k group][column] order, which would fall in one bank; the
// column is XOR-ed with the k group so that they spread over eight 16-byte
// slots.  The operand reads (one k group, 32 consecutive columns) then read
// a permutation of those columns, still without conflict.  The fast path
// stores whole k-group rows and keeps the plain order.
template <int PATH>
__device__ __forceinline__ int b_col(int cg, int c) {
  return PATH == 0 ? c : (c ^ cg);
}

// The wavefront's A region: 32 token rows of 8 pieces, padded to 9 so that
// the 16 rows read by a quarter-wave fall in different banks.
constexpr int kOutArow = 9;

template <int PATH>
__device__ __forceinline__ void out_store(const OutStage<PATH> &st, u32x4_t (*Bs)[64], u32x4_t *As) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (PATH == 0)
    Bs[tid >> 6][tid & 63] = st.b;
  else
    Bs[tid & 7][b_col<PATH>(tid & 7, tid >> 3)] = st.b;
  wave_lds_fence();  // the previous chunk's reads of As are done
#pragma unroll
  for (int q = 0; q < OutStage<PATH>::NA; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) As[(q * kOutTok + i * 8 + (lane >> 3)) * kOutArow + (lane & 7)] = st.a[q][i];
}

template <int PATH>
__device__ __forceinline__ void out_mma(const u32x4_t (*Bs)[64], const u32x4_t *As, f32x16_t (&acc)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int cg = ks * 2 + (lane >> 5);
    const bf16x8_t b0 = as_bf16x8(Bs[cg][b_col<PATH>(cg, lane & 31)]);
    const bf16x8_t b1 = as_bf16x8(Bs[cg][b_col<PATH>(cg, 32 + (lane & 31))]);
#pragma unroll
    for (int q = 0; q < OutStage<PATH>::NA; ++q) {
      const bf16x8_t A = as_bf16x8(As[(q * kOutTok + (lane & 31)) * kOutArow + ks * 2 + (lane >> 5)]);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b1, acc[1], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Outputs of a path with at most kThin tokens: streaming the matrix by rows.
//
// With few tokens the output GEMM is a stream of W (slow) or M (fast) and is
// bound by HBM.  A row block is 16 RT output rows (RT tiles of 16), run by
// four wavefronts (half of the output kernel's workgroup) that take a
// quarter of K each and meet in LDS at the end, so there is no barrier in
// the K loop.  v_mfma_f32_16x16x32_bf16 with A = 16 matrix rows and B = 16
// tokens (kThin tokens are two B groups).  Every row block reads all of the
// path's token rows, so more rows per block means fewer token bytes per
// matrix byte: with 32 rows (the slow path) the CUs take in one byte of x
// per byte of W (with 16 rows, two).
//
// In the MFMA operand layout the 16 lanes of a quarter-wave hold 16 different
// rows, so loading W rows or token rows in that layout touches 16 cache lines
// per quarter-wave and the address unit, not HBM, sets the pace.  Each
// wavefront therefore loads a stage (4 k-steps = 128 columns of K) with
// row-contiguous 16-byte pieces (16 lanes cover 256 bytes of one row), writes
// it to its own LDS region and reads it back in operand layout.  The image M
// is stored in operand order already (64 rows x 16 bytes contiguous) and is
// read directly.  One stage is in flight in registers while the previous one
// goes through LDS and the matrix cores.
// ---------------------------------------------------------------------------
#ifndef GSI_THIN_RT_SLOW
#define GSI_THIN_RT_SLOW 2
#endif
#ifndef GSI_THIN_RT_FAST
#define GSI_THIN_RT_FAST 1
#endif

template <int PATH>
struct ThinStage {
  static constexpr int NB = PATH == 0 ? 2 : 1;  // B matrices: (g hi, g lo) or (x)
  // 16-row tiles of a row block (the fast path's two B matrices leave no
  // registers for a second tile at two wavefronts per SIMD)
  static constexpr int RT = PATH == 0 ? GSI_THIN_RT_FAST : GSI_THIN_RT_SLOW;
  static constexpr int kRows = 16 * RT;  // output rows of a row block
  u32x4_t A[RT][4];  // slow: piece i * 64 + lane of row tile t (16 x 256 bytes); fast: k-step i of tile t of M
  u32x4_t B[NB][8];  // piece i * 64 + lane of the 32 x 256-byte token tile
};

template <int PATH>
struct ThinLds {
  static constexpr int NB = ThinStage<PATH>::NB;
  static constexpr int kRowA = PATH == 1 ? ThinStage<PATH>::kRows : 0;
  // pieces of 16 bytes, rows padded by one piece so that the 16 rows read by a
  // quarter-wave fall in different banks
  static constexpr int kA = kRowA * 17;
  static constexpr int kPieces = kA + NB * 32 * 17;
};

template <int PATH>
__device__ __forceinline__ void thin_load(ThinStage<PATH> &st, const BArgs &a, int step0, int kend,
                                          int r0, const int (&tk)[8], const u32x4_t *zero) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < ThinStage<PATH>::RT; ++t) {
    if (PATH == 0) {
      const int q = lane >> 4, row = r0 + 16 * t + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kg = (step0 + j) * 32 + 8 * q;
        const bool ok = kg < kend && row < a.d_out;
        const u32x4_t *p = static_cast<const u32x4_t *>(a.M) +
                           ((size_t)(row / 64) * (a.k / 8) + kg / 8) * 64 + (row & 63);
        st.A[t][j] = *(ok ? p : zero);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = i * 64 + lane;
        const int row = r0 + 16 * t + (pc >> 4), kg = step0 * 32 + (pc & 15) * 8;
        const bool ok = kg < kend && row < a.d_out;
        const u32x4_t *p =
            reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.W) + (size_t)row * a.d + kg);
        st.A[t][i] = *(ok ? p : zero);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = tk[i], kg = step0 * 32 + (lane & 15) * 8;
    const bool ok = kg < kend && tok >= 0;
    if (PATH == 0) {
      const size_t off = (size_t)tok * a.kpad + kg;
      st.B[0][i] = *(ok ? reinterpret_cast<const u32x4_t *>(a.ghi + off) : zero);
      st.B[ThinStage<PATH>::NB - 1][i] = *(ok ? reinterpret_cast<const u32x4_t *>(a.glo + off) : zero);
    } else {
      const size_t off = (size_t)tok * a.d + kg;
      st.B[0][i] = *(ok ? reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.x) + off) : zero);
    }
  }
}

template <int PATH>
__device__ __forceinline__ void thin_consume(const ThinStage<PATH> &st, u32x4_t *lds,
                                             f32x4_t (&acc)[ThinStage<PATH>::RT][2]) {
  constexpr int NB = ThinStage<PATH>::NB;
  constexpr int kA = ThinLds<PATH>::kA;
  const int lane = threadIdx.x & 63;
  wave_lds_fence();  // the previous stage's reads are done before it is overwritten
  if (PATH == 1) {
#pragma unroll
    for (int t = 0; t < ThinStage<PATH>::RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pc = i * 64 + lane;
        lds[(16 * t + (pc >> 4)) * 17 + (pc & 15)] = st.A[t][i];
      }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = i * 64 + lane;
      lds[kA + b * 32 * 17 + (pc >> 4) * 17 + (pc & 15)] = st.B[b][i];
    }
  wave_lds_fence();
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t B[2][NB];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int b = 0; b < NB; ++b) B[g][b] = lds[kA + b * 32 * 17 + (16 * g + r) * 17 + 4 * j + q];
#pragma unroll
    for (int t = 0; t < ThinStage<PATH>::RT; ++t) {
      const u32x4_t A = PATH == 1 ? lds[(16 * t + r) * 17 + 4 * j + q] : st.A[t][j];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A), as_bf16x8(B[g][b]), acc[t][g], 0, 0, 0);
    }
  }
}

constexpr int kThinPieces = ThinLds<0>::kPieces > ThinLds<1>::kPieces ? ThinLds<0>::kPieces : ThinLds<1>::kPieces;
static_assert(kThinPieces * 16 >= ThinStage<0>::RT * 2 * 4 * 64 * 4 && kThinPieces * 16 >= ThinStage<1>::RT * 2 * 4 * 64 * 4,
              "the final sums reuse a wavefront's region");

template <int PATH>
__device__ __forceinline__ void bthin_path(const BArgs &a, u32x4_t (*lds)[kThinPieces], const int *toks,
                                           int rb) {
  // four wavefronts (a workgroup of kBlock threads, or one half of the
  // output kernel's eight, each half on its own row block: both halves
  // pass the same barriers)
  const int tid = threadIdx.x & (kBlock - 1);
  const int wave = tid >> 6, lane = tid & 63;
  const int r0 = rb * ThinStage<PATH>::kRows;
  // one zero piece per lane (a uniform fallback address becomes a branch)
  const u32x4_t *zero = static_cast<const u32x4_t *>(a.zeros) + (lane & 15);
  const int K = PATH == 0 ? a.kpad : a.d;
  const int steps = (K + 31) / 32;  // k-steps of 32
  const int per = (steps + kWaves - 1) / kWaves;
  const int s0 = wave * per;
  const int s_end = min(steps, s0 + per);
  const int kend = min(s_end * 32, PATH == 0 ? a.k : a.d);  // this wavefront's K ends here

  int tk[8];  // token of each of this lane's 16-byte pieces of the token tile
#pragma unroll
  for (int i = 0; i < 8; ++i) tk[i] = toks[(i * 64 + lane) >> 4];

  f32x4_t acc[ThinStage<PATH>::RT][2];
#pragma unroll
  for (int t = 0; t < ThinStage<PATH>::RT; ++t)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[t][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  ThinStage<PATH> sa, sb;
  thin_load<PATH>(sa, a, s0, kend, r0, tk, zero);
  for (int st = s0; st < s_end; st += 8) {
    thin_load<PATH>(sb, a, st + 4, kend, r0, tk, zero);
    thin_consume<PATH>(sa, lds[wave], acc);
    thin_load<PATH>(sa, a, st + 8, kend, r0, tk, zero);
    thin_consume<PATH>(sb, lds[wave], acc);
  }
  // partial sums of the four K quarters, through each wavefront's own region:
  // element ((t * 2 + g) * 4 + i) * 64 + lane
  wave_lds_fence();
  float *red = reinterpret_cast<float *>(lds[wave]);
#pragma unroll
  for (int t = 0; t < ThinStage<PATH>::RT; ++t)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((t * 2 + g) * 4 + i) * 64 + lane] = acc[t][g][i];
  __syncthreads();
  uint16_t *Y = static_cast<uint16_t *>(a.y);
#pragma unroll
  for (int h = 0; h < 2 * ThinStage<PATH>::RT; ++h) {
    const int e = tid + h * kBlock;  // (tile, group, element, lane)
    const int t = e >> 9, g = (e >> 8) & 1, i = (e >> 6) & 3, l = e & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += reinterpret_cast<const float *>(lds[w])[e];
    const int tok = toks[g * 16 + (l & 15)];
    const int r = r0 + 16 * t + 4 * (l >> 4) + i;
    if (tok >= 0 && r < a.d_out) Y[(size_t)tok * a.d_out + r] = f2bf(v);
  }
  __syncthreads();  // every wavefront's region is free again
}

// LDS of the wide kernel, sized for the fast path (two A matrices); the
// fast items of wide_fast_item use Bs and As as one block.
struct OutLds {
  union {
    struct {
      u32x4_t Bs[2][8][64];                          // double-buffered 64-wide K chunk: [k group][column]
      u32x4_t As[kOutWaves][2 * kOutTok * kOutArow];  // each wavefront's A chunk
    };
    u32x4_t thin[2 * kWaves][kThinPieces];  // row-stream regions (two halves of four wavefronts)
  };
  int16_t idx[kMaxBatch];  // tokens of both paths (path_lists)
  int2 scan[kOutWaves];    // wavefront totals of the compaction scan
  int toks[2][kThin];      // tokens of each path with 1 to kThin tokens (-1: none)
};

template <int PATH>
__device__ __forceinline__ void bout_path(const BArgs &a, OutLds &L, int tile, const int16_t *idx,
                                          int count) {
  auto &Bs = L.Bs;
  auto &As = L.As;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int o0 = tile * 64;
  // one zero piece per lane (a uniform fallback address becomes a branch)
  const u32x4_t *zero = static_cast<const u32x4_t *>(a.zeros) + (lane & 15);

  const int K = PATH == 0 ? a.kpad : a.d;
  const int nch = (K + 63) / 64;
  uint16_t *Y = static_cast<uint16_t *>(a.y);

  for (int base = 0; base < count; base += kOutRound) {
    // A wavefront with no token in this round (fewer than 256 tokens left)
    // still loads and stores its share of every B chunk and keeps the
    // barriers, but skips the products.
    const int row0 = base + wave * kOutTok;
    const bool has_tokens = row0 < count;
    int tk[4];  // token of each of this lane's A pieces
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + i * 8 + (lane >> 3);
      tk[i] = row < count ? idx[row] : -1;
    }
    f32x16_t acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;

    // A ring of D stages: chunk i is consumed while chunks i+1 .. i+D-1
    // load (two stages: with two wavefronts per SIMD, three or four measured
    // no faster).  The ring is indexed by constants only (every loop over it
    // is unrolled), so it stays in registers; loads past K read the zero block.
    constexpr int D = OutStage<PATH>::kDepth;
    OutStage<PATH> st[D];
#pragma unroll
    for (int j = 0; j + 1 < D; ++j) out_load<PATH>(st[j], a, j * 64, o0, tk, zero);
    int i = 0;
    for (; i + D <= nch; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        out_load<PATH>(st[(j + D - 1) % D], a, (i + j + D - 1) * 64, o0, tk, zero);
        out_store<PATH>(st[j], Bs[(i + j) & 1], As[wave]);
        __syncthreads();
        if (has_tokens) out_mma<PATH>(Bs[(i + j) & 1], As[wave], acc);
      }
    }
#pragma unroll
    for (int j = 0; j + 1 < D; ++j) {
      if (i + j < nch) {
        out_store<PATH>(st[j], Bs[(i + j) & 1], As[wave]);
        __syncthreads();
        if (has_tokens) out_mma<PATH>(Bs[(i + j) & 1], As[wave], acc);
      }
    }
    __syncthreads();
    // The wavefront's 32 tokens x 64 columns of y go through its own LDS
    // region (free after the loop), so that each lane stores 16-byte pieces
    // of token rows instead of single elements.
    constexpr int kYrow = 72;  // bf16 per staged row: 64 columns, padded to a 16-byte multiple
    uint16_t *yt = reinterpret_cast<uint16_t *>(As[wave]);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        yt[r * kYrow + c * 32 + (lane & 31)] = f2bf(acc[c][e]);
      }
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pc = q * 64 + lane;  // piece: staged row pc / 8, columns 8 (pc % 8) ..
      const int r = pc >> 3, c8 = (pc & 7) * 8;
      const int row = row0 + r;
      if (row < count && o0 + c8 < a.d_out)
        *reinterpret_cast<u32x4_t *>(Y + (size_t)idx[row] * a.d_out + o0 + c8) =
            *reinterpret_cast<const u32x4_t *>(yt + r * kYrow + c8);
    }
    wave_lds_fence();  // the next round's stores to this region come after these reads
  }
}

// ---------------------------------------------------------------------------
// Wide fast path (more than kThin fast tokens): Y_f = G_f M^T with g as the
// two bf16 planes hi + lo.  K is small (k <= 1024), so an item is built to
// have all of its loads in flight in a few rounds, not one round per 64 of
// k.  An item is 64 fast tokens x 256 output rows: each of the eight
// wavefronts owns 32 rows (one MFMA column block of a 64-row image tile)
// for the 64 tokens (two 32-row blocks), v_mfma_f32_32x32x16_bf16.  The
// tiled image is already in B-operand order (32 lanes read 512 contiguous
// bytes of one k group), so M goes straight into registers, eight k-steps
// of 16 per stage, the next stage in flight while one is multiplied.  g's
// planes for the 64 tokens go through LDS 256 of k per pass (coalesced
// 512-byte token rows), stored as [plane][k group][token ^ k group] so that
// the stores and the operand reads (32 consecutive tokens of one k group)
// spread over the banks.
// ---------------------------------------------------------------------------
constexpr int kWideTok = 64;                    // fast tokens of an item
constexpr int kWideRows = kOutWaves * 32;       // output rows of an item
constexpr int kWideKc = 256;                    // k of g per LDS pass
constexpr int kWideStage = 8;                   // k-steps of 16 per register stage of M
constexpr int kWideStagesPerPass = kWideKc / 16 / kWideStage;
struct WideLds {
  u32x4_t A[2][kWideKc / 8][kWideTok];  // [plane][k group][token ^ k group]
};
static_assert(kWideStagesPerPass == 2, "a pass of g spans the two stages of the ring");

__device__ __forceinline__ void wide_load_b(u32x4_t (&b)[kWideStage], const BArgs &a, int tile, int cb,
                                            int tiles, int step0, const u32x4_t *zero) {
  const int lane = threadIdx.x & 63;
  const int kg8 = a.k / 8;
#pragma unroll
  for (int s = 0; s < kWideStage; ++s) {
    const int q = 2 * (step0 + s) + (lane >> 5);  // k group of this lane
    const bool ok = tile < tiles && q < kg8;
    b[s] = *(ok ? static_cast<const u32x4_t *>(a.M) + ((size_t)tile * kg8 + q) * 64 + cb * 32 + (lane & 31)
                : zero);
  }
}

__device__ __forceinline__ void wide_mma(const u32x4_t (&b)[kWideStage], const WideLds &L, int step0, int steps,
                                         f32x16_t (&acc)[2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < kWideStage; ++s) {
    if (step0 + s < steps) {
      const int q = 2 * ((step0 + s) % (kWideKc / 16)) + (lane >> 5);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int m = tb * 32 + (lane & 31);
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(L.A[0][q][m ^ q]), as_bf16x8(b[s]), acc[tb], 0,
                                                          0, 0);
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(L.A[1][q][m ^ q]), as_bf16x8(b[s]), acc[tb], 0,
                                                          0, 0);
      }
    }
  }
}

// g's planes of tokens list[0..count) (count <= 64), k in [kc0, kc0 + 256),
// into L.A (zero outside the tokens and from kpad on).  Every thread issues
// its loads before its first store.
__device__ __forceinline__ void wide_stage_a(WideLds &L, const BArgs &a, const int16_t *list, int count, int kc0,
                                             const u32x4_t *zero) {
  constexpr int kGroups = kWideKc / 8;
  constexpr int kPieces = 2 * kGroups * kWideTok / kOutThreads;  // 8 per thread
  const int tid = threadIdx.x;
  u32x4_t v[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int p = tid + i * kOutThreads;
    const int plane = p / (kGroups * kWideTok), rem = p % (kGroups * kWideTok);
    const int m = rem / kGroups, q = rem % kGroups;
    const int kk = kc0 + 8 * q;
    const bool ok = m < count && kk < a.kpad;
    const uint16_t *src = plane == 0 ? a.ghi : a.glo;
    v[i] = *(ok ? reinterpret_cast<const u32x4_t *>(src + (size_t)list[ok ? m : 0] * a.kpad + kk) : zero);
  }
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int p = tid + i * kOutThreads;
    const int plane = p / (kGroups * kWideTok), rem = p % (kGroups * kWideTok);
    const int m = rem / kGroups, q = rem % kGroups;
    L.A[plane][q][m ^ q] = v[i];
  }
}

// One item: fast tokens list[0..count) (count <= 64) x output rows
// [256 rg, 256 rg + 256).  lds: at least sizeof(WideLds) bytes.
__device__ __forceinline__ void wide_fast_item(const BArgs &a, unsigned char *lds, const int16_t *list, int count,
                                               int rg) {
  WideLds &L = *reinterpret_cast<WideLds *>(lds);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const u32x4_t *zero = static_cast<const u32x4_t *>(a.zeros) + (lane & 15);
  const int tiles = (a.d_out + 63) / 64;
  const int tile = rg * (kWideRows / 64) + (wave >> 1), cb = wave & 1;
  const int steps = a.kpad / 16;  // k-steps of 16
  const int nstage = (steps + kWideStage - 1) / kWideStage;
  f32x16_t acc[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tb][i] = 0.f;
  u32x4_t b0[kWideStage], b1[kWideStage];
  wide_load_b(b0, a, tile, cb, tiles, 0, zero);
  // stages g (b0) and g + 1 (b1) make one pass of g's planes
  for (int g = 0; g < nstage; g += 2) {
    __syncthreads();  // the previous pass's operand reads are done
    wide_stage_a(L, a, list, count, (g / kWideStagesPerPass) * kWideKc, zero);
    __syncthreads();
    if (g + 1 < nstage) wide_load_b(b1, a, tile, cb, tiles, (g + 1) * kWideStage, zero);
    wide_mma(b0, L, g * kWideStage, steps, acc);
    if (g + 1 < nstage) {
      if (g + 2 < nstage) wide_load_b(b0, a, tile, cb, tiles, (g + 2) * kWideStage, zero);
      wide_mma(b1, L, (g + 1) * kWideStage, steps, acc);
    }
  }
  // y through LDS: each wavefront's 64 tokens x 32 rows as bf16 rows of 40
  // (padded), then 16-byte pieces of token rows
  __syncthreads();  // every wavefront is done with L.A
  constexpr int kYrow = 40;
  uint16_t *yt = reinterpret_cast<uint16_t *>(lds) + wave * kWideTok * kYrow;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = tb * 32 + 8 * (i / 4) + 4 * (lane >> 5) + (i & 3);
      yt[m * kYrow + (lane & 31)] = f2bf(acc[tb][i]);
    }
  wave_lds_fence();
  uint16_t *Y = static_cast<uint16_t *>(a.y);
  const int o0 = tile * 64 + cb * 32;
#pragma unroll
  for (int q = 0; q < kWideTok * 4 / 64; ++q) {
    const int pc = q * 64 + lane;  // piece: token pc / 4, rows 8 (pc % 4) ..
    const int m = pc >> 2, c8 = (pc & 3) * 8;
    if (m < count && tile < tiles && o0 + c8 < a.d_out)
      *reinterpret_cast<u32x4_t *>(Y + (size_t)list[m] * a.d_out + o0 + c8) =
          *reinterpret_cast<const u32x4_t *>(yt + m * kYrow + c8);
  }
  __syncthreads();  // the staged rows are read before the LDS is reused
}

// Every output of the call in one launch: the workgroups (one per CU) walk
// the row-stream items of the paths with 1 to kThin tokens (pairs of row
// blocks, one per half of the workgroup), then the wide items of the paths
// with more (the fast path in items of 64 tokens x 256 rows, the slow
// path's 64-column tiles).  A call with both kinds of path thus runs them in
// one launch.  Each role is walked in a loop of its own over the
// workgroup's items (blockIdx.x, + gridDim.x, ...): within one loop the
// registers each role keeps for its items would be live across the other's,
// which does not fit (the roles use up to all 256).  With no work the workgroups leave after the
// compaction.
__global__ void __launch_bounds__(kOutThreads, 1) bout_kernel(BArgs a) {
  __shared__ __align__(16) OutLds L;
  static_assert(sizeof(WideLds) <= sizeof(L.Bs) + sizeof(L.As) &&
                    kOutWaves * kWideTok * 40 * 2 <= sizeof(L.Bs) + sizeof(L.As),
                "the fast items use Bs and As as one block");
  static_assert(kOutWaves == 2 * kWaves, "the row streams run as two halves of four wavefronts");
  const int tid = threadIdx.x;
  const int2 cnt = path_lists<kOutThreads>(a, L.idx, L.scan);
  if (tid < 2 * kThin) {
    const int p = tid / kThin, i = tid % kThin;
    const int c = p == 0 ? cnt.x : cnt.y;
    L.toks[p][i] = i < c ? L.idx[(p == 0 ? 0 : cnt.x) + i] : -1;
  }
  __syncthreads();
  // row-stream items: pairs of row blocks (a block past d_out reads zeros
  // and writes nothing), fast path first
  const int bf = (cnt.x > 0 && cnt.x <= kThin) ? (a.d_out + ThinStage<0>::kRows - 1) / ThinStage<0>::kRows : 0;
  const int bs = (cnt.y > 0 && cnt.y <= kThin) ? (a.d_out + ThinStage<1>::kRows - 1) / ThinStage<1>::kRows : 0;
  const int pf = (bf + 1) / 2;
  const int nt = pf + (bs + 1) / 2;
  // wide items
  const int tiles = (a.d_out + 63) / 64;
  const int rgs = (a.d_out + kWideRows - 1) / kWideRows;
  const int nf = cnt.x > kThin ? ((cnt.x + kWideTok - 1) / kWideTok) * rgs : 0;
  const int ns = cnt.y > kThin ? tiles : 0;
  const int half = tid / kBlock;
  int it = blockIdx.x;
  for (; it < nt; it += gridDim.x) {
    if (it < pf)
      bthin_path<0>(a, L.thin + kWaves * half, L.toks[0], 2 * it + half);
    else
      bthin_path<1>(a, L.thin + kWaves * half, L.toks[1], 2 * (it - pf) + half);
  }
  for (; it < nt + nf; it += gridDim.x) {
    const int jt = it - nt, tr = jt / rgs;
    wide_fast_item(a, reinterpret_cast<unsigned char *>(&L.Bs[0][0][0]), L.idx + tr * kWideTok,
                   min(kWideTok, cnt.x - tr * kWideTok), jt % rgs);
  }
  for (; it < nt + nf + ns; it += gridDim.x) bout_path<1>(a, L, it - nt - nf, L.idx + cnt.x, cnt.y);
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
      // swizzled by column group as in the projection GEMM (bank spread)
      const int rs = r ^ (8 * cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[cg * 8 + e][rs] = h[e];
    }
    __syncthreads();
    for (int kk = 0; kk < rows; kk += 32) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok && kk + kq < rows) u = *reinterpret_cast<const uint4 *>(W + (size_t)o * d + i0 + kk + kq);
      const bf16x8_t A = as_bf16x8(u);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = c * 16 + (lane & 15);
        const uint4 b = *reinterpret_cast<const uint4 *>(&Vt[col][(kk + kq) ^ (8 * (col >> 3))]);
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
  // one output launch: about one workgroup per CU (the LDS of the row
  // streams leaves room for one), looping over the items of both paths
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  hipLaunchKernelGGL(bout_kernel, dim3(cus), dim3(kOutThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gsi
