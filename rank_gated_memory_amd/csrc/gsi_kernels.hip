// HIP kernels of the gated subspace linear map for gfx950 (CDNA4, wave64).
//
// Method: "Gated Subspace Inference for Transformer Acceleration"
// (S. J. Thomas, 2026), technical summary (GSI-TS) §2.1-§2.2.
//
// Batch-1 path (one token per call, many calls per launch).  Work comes in
// units: a projection unit is a row chunk of one call's V_k (partial
// g = V_k^T x and partial ||x||^2, fp32), an output unit a run of 64-row
// tiles of M (fast, y = M g) or of rows of W (slow, y = W x).  V_k, M and W
// are streamed with nontemporal 16-byte loads.
//
//   stack_kernel : gsi_stack, one persistent launch per stack.  Workgroups
//                  take projection and output tickets wave by wave (from
//                  eight group counters; at the end of a wave, output
//                  tickets from whichever group has most left).  The
//                  workgroup that writes a call's last partial sums the
//                  partials in a fixed order (bitwise deterministic; in two
//                  levels of at most 64 rows for calls with many units),
//                  forms ||g||^2, rho and the gate (GSI-TS §2.2) and appends
//                  the call to the wave's open list; output units of open
//                  calls run while other calls still project (latency-bound
//                  waves number their output tickets statically instead and
//                  publish each gate in a word of its own).  A wave is
//                  entered once every workgroup has left the previous one
//                  (per-group counters and ready flags), so a call may read
//                  the y of an earlier wave.  Every device-side wait is
//                  bounded and reports through a status word.
//   proj_kernel  : the projection phase as its own launch (gsi_stack_phase,
//   apply_kernel   and gsi_linear's single-map path), then the output phase:
//                  the projection launch leaves a prefix over calls of the
//                  units their chosen paths need, and apply_kernel's
//                  workgroups take contiguous, equal shares of those units.
//
// Cross-XCD hand-off without cache maintenance: the eight XCDs of gfx950 have
// private L2s, and an agent-scope fence compiles to an L2 write-back +
// invalidate that costs ~10x the whole projection when every workgroup
// issues one.  So partials, g, control words and the activations handed
// between waves are written with agent-scope atomic stores (write-through,
// "sc1"), each thread waits for its stores to be acknowledged (s_waitcnt 0)
// before the workgroup barrier that precedes the publishing atomic, and the
// readers use agent-scope atomic loads (which bypass stale L2 lines).
//
// Fast units read the tiled image M (gsi.h) in 16-byte vectors against g in
// LDS, one lane per output row (one tile split over the four wavefronts in
// latency-bound waves); slow units take one wavefront per row of W with x
// staged in LDS and a wave reduction.
// prepare_kernel: M = W V_k for fp32 maps (FMA, LDS tiled), written in the
//                 tiled layout described in gsi.h (bf16 maps use the MFMA
//                 kernel in gsi_batched.hip).
#include <hip/hip_runtime.h>

#include <cfloat>

#include "gsi_gram.h"
#include "gsi_internal.h"

namespace gsi {

// Per-job trace of stack_kernel, compiled only into the instrumented build
// (-DGSI_TRACE=1; build.build_traced): thread 0 of each workgroup writes one
// record per job into the workgroup's own slots (no shared counter, so
// recording adds no contended atomics), {start, end, block << 32 | kind << 8
// | slow, call << 32 | unit}, with times from the 100 MHz constant clock.
// kind: 1 projection unit, 2 output unit (in a wave with static output
// tickets: from the ticket's first loads, including the wait for the gate),
// 7 leaving the job loop, 8 choosing the next job (including any wait for a
// gate or a wave), 9 workgroup start, 10 a static output ticket left void by
// its gate;
// unused slots stay zero.  A unit's end is taken after its memory operations
// completed (s_waitcnt 0), which the product build does not wait for.  Read
// back with gsi_trace_read, cleared with gsi_trace_reset (extern "C",
// instrumented build only).
#ifndef GSI_TRACE
#define GSI_TRACE 0
#endif
#if GSI_TRACE
constexpr unsigned kTraceBlocks = 1024;  // workgroups traced (by index)
constexpr unsigned kTracePer = 512;      // records per workgroup
__device__ unsigned long long g_trace[4ull * kTraceBlocks * kTracePer];
__device__ __forceinline__ void trace_rec(unsigned &n, unsigned long long t0, unsigned long long t1, int kind,
                                          int c, int u, int slow) {
  if (blockIdx.x < kTraceBlocks && n < kTracePer) {
    unsigned long long *r = g_trace + 4ull * (blockIdx.x * kTracePer + n);
    r[0] = t0;
    r[1] = t1;
    r[2] = ((unsigned long long)blockIdx.x << 32) | ((unsigned long long)kind << 8) | (unsigned)slow;
    r[3] = ((unsigned long long)(unsigned)c << 32) | (unsigned)u;
  }
  ++n;
}
#define GSI_TRACE_ONLY(...) __VA_ARGS__
#else
#define GSI_TRACE_ONLY(...)
#endif

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ uint16_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                             // nearest-even
  return (uint16_t)(u >> 16);
}

template <typename T>
struct Vec;

template <>
struct Vec<float> {
  static constexpr int VW = 4;
  static constexpr int ESIZE = 4;
  __device__ __forceinline__ static void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static float load1(const void *p, size_t i) {
    return static_cast<const float *>(p)[i];
  }
  __device__ __forceinline__ static void store1(void *p, size_t i, float v) {
    static_cast<float *>(p)[i] = v;
  }
  // agent-coherent forms (data handed between waves of one launch)
  __device__ __forceinline__ static float load1c(const void *p, size_t i) {
    return __hip_atomic_load(const_cast<float *>(static_cast<const float *>(p)) + i,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ static void store1c(void *p, size_t i, float v) {
    __hip_atomic_store(static_cast<float *>(p) + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

template <>
struct Vec<bf16_t> {
  static constexpr int VW = 8;
  static constexpr int ESIZE = 2;
  __device__ __forceinline__ static void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
  __device__ __forceinline__ static float load1(const void *p, size_t i) {
    return __uint_as_float((uint32_t) static_cast<const uint16_t *>(p)[i] << 16);
  }
  __device__ __forceinline__ static void store1(void *p, size_t i, float v) {
    static_cast<uint16_t *>(p)[i] = float_to_bf16(v);
  }
  __device__ __forceinline__ static float load1c(const void *p, size_t i) {
    const uint16_t b = __hip_atomic_load(const_cast<uint16_t *>(static_cast<const uint16_t *>(p)) + i,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __uint_as_float((uint32_t)b << 16);
  }
  __device__ __forceinline__ static void store1c(void *p, size_t i, float v) {
    __hip_atomic_store(static_cast<uint16_t *>(p) + i, float_to_bf16(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Streaming 16-byte loads of data read once per launch (V_k, M and W rows):
// marked nontemporal so that they do not displace the lines that are
// reused.  On this part a chunked streaming read reaches ~7.2 TB/s this way
// against ~6.3 TB/s with ordinary loads.
#ifndef GSI_NT_LOADS
#define GSI_NT_LOADS 1
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
#if GSI_NT_LOADS
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
#else
  return *p;
#endif
}

// One element of y: agent-coherent when a later wave of the same launch reads it.
template <typename T>
__device__ __forceinline__ void store_y(const CallDesc &cd, int i, float v) {
  if (cd.flags & kCallYCoherent)
    Vec<T>::store1c(cd.y, i, v);
  else
    Vec<T>::store1(cd.y, i, v);
}

__device__ __forceinline__ float wave_sum(float v) {
  // Butterfly: every lane ends with the same, order-fixed sum.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup; every thread returns the same value.
__device__ __forceinline__ float block_sum(float v, float *sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += sh[i];
  return t;
}

// rho from ||x||^2 and ||g||^2 (exact for an orthonormal basis).
// ||x|| = 0 gives 0; a non-finite norm gives NaN so that the gate sends the
// token down the slow path.
__device__ __forceinline__ float rho_from_norms(float xx, float gg) {
  if (!(xx <= FLT_MAX) || !(gg <= FLT_MAX)) return __builtin_nanf("");
  if (xx == 0.f) return 0.f;
  const float t = 1.f - gg / xx;
  return t > 0.f ? sqrtf(t) : 0.f;
}

// Agent-coherent accesses used for the partials handed between workgroups.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ CallDesc load_call(const KArgs &a, int c) {
  if (a.table) return a.table[c];
  CallDesc d = a.one;
  d.x = static_cast<const char *>(a.one.x) + (int64_t)c * a.x_stride;
  d.y = static_cast<char *>(a.one.y) + (int64_t)c * a.y_stride;
  if (d.rho) d.rho += c;
  if (d.slow) d.slow += c;
  d.a_begin = c * a.one.a_units;
  d.part_off = a.one.part_off +
               (int64_t)c * ((int64_t)(a.one.a_units + (a.one.groups > 1 ? a.one.groups : 0)) * (a.one.k + 4));
  d.g_off = a.one.g_off + (int64_t)c * ((a.one.k + 3) / 4 * 4);
  d.gate_off = c;
  return d;
}

// ---------------------------------------------------------------------------
// Projection: partial g and ||x||^2 per row chunk, gate by the last chunk.
// MODE is the gsi_mode (a template argument so that each mode is a distinct
// kernel in traces).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_coherent_i(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent_i(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of need[0..n) into pref[0..n] by one workgroup (the last
// call to finish its gate); need[] is read with agent-coherent loads.
__device__ void launch_prefix(const KArgs &a, int *sh_int) {
  const int tid = threadIdx.x;
  const int n = a.n;
  const int per = (n + kBlock - 1) / kBlock;  // calls per thread (n <= kMaxCalls)
  const int c0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (c0 + i < n) local += load_coherent_i(a.need + c0 + i);
  sh_int[tid] = local;
  __syncthreads();
  for (int off = 1; off < kBlock; off <<= 1) {
    const int t = tid >= off ? sh_int[tid - off] : 0;
    __syncthreads();
    sh_int[tid] += t;
    __syncthreads();
  }
  int run = sh_int[tid] - local;  // exclusive prefix at c0
  for (int i = 0; i < per; ++i) {
    if (c0 + i < n) {
      a.pref[c0 + i] = run;
      run += load_coherent_i(a.need + c0 + i);
    }
  }
  if (tid == kBlock - 1) a.pref[n] = sh_int[kBlock - 1];
}

// Partial g = V_k^T x and ||x||^2 over projection unit q of a call (a chunk
// of a_rows rows of V_k), written to `part` ([k] then ||x||^2) with
// agent-coherent stores.  XC: x is read with agent-coherent loads.
template <typename T, int UNROLL, bool XC>
__device__ __forceinline__ void proj_partial(const CallDesc &cd, int q, float *part, float *red,
                                             float *sh) {
  constexpr int VW = Vec<T>::VW;
  const int tid = threadIdx.x;
  const int row0 = q * cd.a_rows;
  const int rows = min(cd.a_rows, cd.d - row0);
  const int k = cd.k;
  const int tpr = k / VW;        // lanes per row of V_k
  const int rpp = kBlock / tpr;  // rows per pass
  const int slot = tid / tpr;
  const int col = tid - slot * tpr;
  const bool active = slot < rpp;
  // Each thread reads the x entry of every V_k row it multiplies (the lanes
  // of a row share the address), so streaming starts without a staging
  // barrier; the column-0 lane of each row also accumulates ||x||^2.
  float xx = 0.f;
  if (active) {
    float acc[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] = 0.f;
    const uint4 *vp =
        reinterpret_cast<const uint4 *>(static_cast<const T *>(cd.V) + (size_t)row0 * k) + col;
    const T *xp = static_cast<const T *>(cd.x) + row0;
    int r = slot;
    // full batches: no branch around any load
    for (; r + (UNROLL - 1) * rpp < rows; r += rpp * UNROLL) {
      uint4 v[UNROLL];
      float xv[UNROLL];
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        v[j] = ld_stream(vp + (size_t)(r + j * rpp) * tpr);
        xv[j] = XC ? Vec<T>::load1c(xp, r + j * rpp) : Vec<T>::load1(xp, r + j * rpp);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        float f[VW];
        Vec<T>::unpack(v[j], f);
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] = fmaf(f[e], xv[j], acc[e]);
        if (col == 0) xx = fmaf(xv[j], xv[j], xx);
      }
    }
    // remainder rows of the last chunk of a call
    for (; r < rows; r += rpp) {
      const uint4 v = ld_stream(vp + (size_t)r * tpr);
      const float xv = XC ? Vec<T>::load1c(xp, r) : Vec<T>::load1(xp, r);
      float f[VW];
      Vec<T>::unpack(v, f);
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[e] = fmaf(f[e], xv, acc[e]);
      if (col == 0) xx = fmaf(xv, xv, xx);
    }
#pragma unroll
    for (int e = 0; e < VW; ++e) red[slot * k + col * VW + e] = acc[e];
  }
  xx = block_sum(xx, sh);  // also publishes red to the workgroup

  for (int j = tid; j < k; j += kBlock) {
    float s = 0.f;
    for (int sl = 0; sl < rpp; ++sl) s += red[sl * k + j];
    store_coherent(part + j, s);
  }
  if (tid == 0) store_coherent(part + k, xx);
}

// Column j of `count` partial rows (stride floats apart) summed in row
// order with agent-coherent loads: batches of 64, then of 16, then one
// predicated batch for the last 1-15 rows, every load of a batch issued
// before its first add (a tail of a few rows costs one round trip, not one
// each).
__device__ __forceinline__ float sum_rows(const float *p0, int count, int stride, int j) {
  float s = 0.f;
  int qq = 0;
  for (; qq + 64 <= count; qq += 64) {
    float t[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) t[i] = load_coherent(p0 + (int64_t)(qq + i) * stride + j);
#pragma unroll
    for (int i = 0; i < 64; ++i) s += t[i];
  }
  for (; qq + 16 <= count; qq += 16) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = load_coherent(p0 + (int64_t)(qq + i) * stride + j);
#pragma unroll
    for (int i = 0; i < 16; ++i) s += t[i];
  }
  if (qq < count) {
    float t[15];
#pragma unroll
    for (int i = 0; i < 15; ++i)
      t[i] = qq + i < count ? load_coherent(p0 + (int64_t)(qq + i) * stride + j) : 0.f;
#pragma unroll
    for (int i = 0; i < 15; ++i)
      if (qq + i < count) s += t[i];
  }
  return s;
}

// Hand-off after a projection unit stored its partial (after s_waitcnt 0
// and a barrier).  Returns 1 on the workgroup that must finish the call:
// with one group, the last unit; with several, the last unit of a group
// first sums its group's partials into the group partial, and the last
// group to do so finishes.  flag: an LDS int.
__device__ __forceinline__ int projection_handoff(const CallDesc &cd, int c, int q, float *wsf,
                                                  uint32_t *counters, uint32_t *gcounters, int *flag) {
  const int tid = threadIdx.x;
  const int stride = cd.k + 4;
  if (cd.groups > 1) {
    const int grp = q / kGroupUnits;
    const int gsize = min(kGroupUnits, cd.a_units - grp * kGroupUnits);
    if (tid == 0)
      *flag = __hip_atomic_fetch_add(gcounters + cd.a_begin + grp, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(gsize - 1) ? 1 : 0;
    __syncthreads();
    if (!*flag) return 0;
    const float *src = wsf + cd.part_off + (int64_t)grp * kGroupUnits * stride;
    float *dst = wsf + cd.part_off + (int64_t)(cd.a_units + grp) * stride;
    for (int j = tid; j <= cd.k; j += kBlock) store_coherent(dst + j, sum_rows(src, gsize, stride, j));
    if (tid == 0) __hip_atomic_store(gcounters + cd.a_begin + grp, 0u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const unsigned last = (unsigned)((cd.groups > 1 ? cd.groups : cd.a_units) - 1);
  if (tid == 0)
    *flag = __hip_atomic_fetch_add(counters + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == last ? 1 : 0;
  __syncthreads();
  return *flag;
}

// The partial rows the finishing workgroup sums: the unit partials, or the
// group partials stored after them.
__device__ __forceinline__ const float *final_rows(const CallDesc &cd, const float *wsf, int *count) {
  if (cd.groups > 1) {
    *count = cd.groups;
    return wsf + cd.part_off + (int64_t)cd.a_units * (cd.k + 4);
  }
  *count = cd.a_units;
  return wsf + cd.part_off;
}

// Run by the workgroup that finishes a call: sums the `count` final partial
// rows at p0 in a fixed order (bitwise deterministic), writes g
// (agent-coherent stores when GC), forms ||x||^2, ||g||^2 and rho
// (GSI-TS §2.2), and clears the call's counter.  With a cached E = V_k^T V_k - I, rho is exact for the
// stored basis (g also goes to the LDS scratch gl, k floats).  Returns
// {rho, ||x||^2, ||g||^2} (valid on thread 0).
template <typename T, bool GC>
__device__ __forceinline__ float3 finish_projection(const CallDesc &cd, const float *p0, int count,
                                                    float *gw, uint32_t *counters, float *sh, float *gl) {
  const int tid = threadIdx.x;
  const int k = cd.k;
  const int stride = k + 4;
  float gg = 0.f;
  for (int j = tid; j < k; j += kBlock) {
    const float s = sum_rows(p0, count, stride, j);
    if (GC)
      store_coherent(gw + j, s);
    else
      gw[j] = s;
    if (cd.G) gl[j] = s;
    gg = fmaf(s, s, gg);
  }
  float xp = 0.f;
  for (int qq = tid; qq < count; qq += kBlock) xp += load_coherent(p0 + (int64_t)qq * stride + k);
  gg = block_sum(gg, sh);
  const float xxt = block_sum(xp, sh);
  if (tid == 0) counters[cd.gate_off] = 0u;  // ready for the next launch on this workspace
  if (cd.G) {
    const float q = gram_quadratic<sizeof(T), kBlock>(cd.G, k, gl, sh);
    return make_float3(rho_exact(xxt, gg, q), xxt, gg);
  }
  return make_float3(rho_from_norms(xxt, gg), xxt, gg);
}

// The gate of one call from its residual ratio (GSI-TS §2.2): slow iff
// !(rho < eps), unless the mode forces a path.  Writes the gate record and
// the caller's rho / slow (thread 0 only) and returns the slow flag.
template <int MODE>
__device__ __forceinline__ int decide_gate(const CallDesc &m, float3 r, void *gate) {
  const int slow = MODE == 2 ? 1 : (MODE == 1 ? 0 : !(r.x < m.eps));
  reinterpret_cast<float4 *>(gate)[m.gate_off] = make_float4(r.x, __int_as_float(slow), r.y, r.z);
  if (m.rho) *m.rho = r.x;
  if (m.slow) *m.slow = (uint8_t)slow;
  return slow;
}

template <typename T, int UNROLL, int MODE>
__global__ void __launch_bounds__(kBlock) proj_kernel(KArgs a) {
  constexpr int VW = Vec<T>::VW;
  __shared__ float red[kBlock * VW];
  __shared__ float sh[kWaves];
  __shared__ int sh_int[kBlock];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int c = a.table ? a.unit_call[u] : (u / a.one.a_units);
  const CallDesc cd = load_call(a, c);
  const int q = u - cd.a_begin;
  proj_partial<T, UNROLL, false>(cd, q, a.wsf + cd.part_off + (int64_t)q * (cd.k + 4), red, sh);

  // Hand the partials over (see the header); the last chunk finishes the gate.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!projection_handoff(cd, cd.gate_off, q, a.wsf, a.counters, a.gcounters, &s_last)) return;

  int rows = 0;
  const float *p0 = final_rows(cd, a.wsf, &rows);
  const float3 r = finish_projection<T, false>(cd, p0, rows, a.wsf + cd.g_off, a.counters, sh, red);
  if (tid == 0) {
    // the gates of this call and of every call sharing its projection
    unsigned members = 0;
    for (int m = c;;) {
      const CallDesc md = m == c ? cd : load_call(a, m);
      const int slow = decide_gate<MODE>(md, r, a.gate);
      store_coherent_i(a.need + m, slow ? md.slow_units : md.fast_units);
      ++members;
      if (md.share_next == 0) break;
      m = md.share_next - 1;
    }
    s_last = (int)members;
  }

  // The last call to finish writes the launch-wide prefix of output units.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned members = (unsigned)s_last;
    const unsigned prev = __hip_atomic_fetch_add(a.counters + a.n, members, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev + members == (unsigned)a.n) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  launch_prefix(a, sh_int);
  if (tid == 0) a.counters[a.n] = 0u;
}

// ---------------------------------------------------------------------------
// Output: fast units (y = M g) and slow units (y = W x) of the chosen paths.
// ---------------------------------------------------------------------------
// Fast unit of one 64-row tile: wavefront w takes the 16-byte column
// vectors w, w + kWaves, ... of every row (one row per lane) and the four
// partial sums meet in LDS (`scr`, kWaves x 64 floats), added in wavefront
// order.  Used by latency-bound waves, where a unit must be small.  The
// first batch of loads is a separate step (fast_tile_load), so that a caller
// can issue it before g is known.
template <typename T, int UNROLL>
__device__ __forceinline__ void fast_tile_load(const CallDesc &cd, int tile, uint4 (&v)[UNROLL]) {
  constexpr int VW = Vec<T>::VW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kv = cd.k / VW;
  const uint4 *m = reinterpret_cast<const uint4 *>(cd.M) + (size_t)tile * kTileRows * kv + lane;
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) {
    const int cg = wave + j * kWaves;
    v[j] = cg < kv ? ld_stream(m + (size_t)cg * kTileRows) : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <typename T, int UNROLL>
__device__ __forceinline__ void fast_tile_finish(const CallDesc &cd, int tile, uint4 (&v)[UNROLL], const float *gs,
                                                 float *scr) {
  constexpr int VW = Vec<T>::VW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kv = cd.k / VW;
  const uint4 *m = reinterpret_cast<const uint4 *>(cd.M) + (size_t)tile * kTileRows * kv + lane;
  float a0 = 0.f, a1 = 0.f;
  for (int cg0 = wave;;) {
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int cg = cg0 + j * kWaves;
      if (cg < kv) {
        float f[VW];
        Vec<T>::unpack(v[j], f);
        const float *gp = gs + cg * VW;
#pragma unroll
        for (int e = 0; e < VW; e += 2) {
          a0 = fmaf(f[e], gp[e], a0);
          a1 = fmaf(f[e + 1], gp[e + 1], a1);
        }
      }
    }
    cg0 += kWaves * UNROLL;
    if (cg0 >= kv) break;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int cg = cg0 + j * kWaves;
      v[j] = cg < kv ? ld_stream(m + (size_t)cg * kTileRows) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  scr[wave * 64 + lane] = a0 + a1;
  __syncthreads();
  if (wave == 0) {
    float t = scr[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += scr[w * 64 + lane];
    const int o = tile * kTileRows + lane;
    if (o < cd.d_out) store_y<T>(cd, o, t);
  }
  __syncthreads();  // scr is free again
}

template <typename T, int UNROLL>
__device__ __forceinline__ void fast_tile_split(const CallDesc &cd, int tile, const float *gs, float *scr) {
  uint4 v[UNROLL];
  fast_tile_load<T, UNROLL>(cd, tile, v);
  fast_tile_finish<T, UNROLL>(cd, tile, v, gs, scr);
}

template <typename T, int UNROLL>
__device__ __forceinline__ void fast_unit(const CallDesc &cd, int local, const float *gs, float *scr) {
  if (cd.fast_tiles == 1) {
    fast_tile_split<T, UNROLL>(cd, local, gs, scr);
    return;
  }
  constexpr int VW = Vec<T>::VW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int tiles = (cd.d_out + kTileRows - 1) / kTileRows;
  const int t1 = min((local + 1) * cd.fast_tiles, tiles);
  const int kv = cd.k / VW;
  const size_t tile_vecs = (size_t)kTileRows * kv;
  // Each wavefront streams two tiles at a time (tiles t and t + kWaves), one
  // output row per lane in each, so 2 * UNROLL 16-byte loads are in flight.
  for (int tile = local * cd.fast_tiles + wave; tile < t1; tile += 2 * kWaves) {
    const bool two = tile + kWaves < t1;
    const uint4 *ma = reinterpret_cast<const uint4 *>(cd.M) + (size_t)tile * tile_vecs + lane;
    const uint4 *mb = ma + (two ? (size_t)kWaves * tile_vecs : 0);
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    for (int cg = 0; cg < kv; cg += UNROLL) {
      uint4 va[UNROLL], vb[UNROLL];
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const bool ok = cg + j < kv;
        va[j] = ok ? ld_stream(ma + (size_t)(cg + j) * kTileRows) : make_uint4(0u, 0u, 0u, 0u);
        vb[j] = (ok && two) ? ld_stream(mb + (size_t)(cg + j) * kTileRows) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        if (cg + j < kv) {
          float fa[VW], fb[VW];
          Vec<T>::unpack(va[j], fa);
          Vec<T>::unpack(vb[j], fb);
          const float *gp = gs + (cg + j) * VW;
#pragma unroll
          for (int e = 0; e < VW; e += 2) {
            a0 = fmaf(fa[e], gp[e], a0);
            a1 = fmaf(fa[e + 1], gp[e + 1], a1);
            b0 = fmaf(fb[e], gp[e], b0);
            b1 = fmaf(fb[e + 1], gp[e + 1], b1);
          }
        }
      }
    }
    const int oa = tile * kTileRows + lane;
    if (oa < cd.d_out) store_y<T>(cd, oa, a0 + a1);
    const int ob = (tile + kWaves) * kTileRows + lane;
    if (two && ob < cd.d_out) store_y<T>(cd, ob, b0 + b1);
  }
}

template <typename T, int UNROLL>
__device__ __forceinline__ void slow_unit(const CallDesc &cd, int local, const uint4 *xs) {
  constexpr int VW = Vec<T>::VW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r0 = local * cd.slow_rows;
  const int r1 = min(r0 + cd.slow_rows, cd.d_out);
  const int nv = cd.d / VW;
  // Each wavefront takes two rows of W at a time (rows r and r + kWaves) so
  // that 2 * UNROLL 16-byte loads per lane are in flight.
  for (int r = r0 + wave; r < r1; r += 2 * kWaves) {
    const bool two = r + kWaves < r1;
    const uint4 *wa = reinterpret_cast<const uint4 *>(static_cast<const T *>(cd.W) + (size_t)r * cd.d);
    const uint4 *wb = wa + (two ? (size_t)kWaves * nv : 0);
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    for (int v0 = lane; v0 < nv; v0 += 64 * UNROLL) {
      uint4 wA[UNROLL], wB[UNROLL];
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int vv = v0 + j * 64;
        wA[j] = vv < nv ? ld_stream(wa + vv) : make_uint4(0u, 0u, 0u, 0u);
        wB[j] = (two && vv < nv) ? ld_stream(wb + vv) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int vv = v0 + j * 64;
        if (vv < nv) {
          float fa[VW], fb[VW], xf[VW];
          Vec<T>::unpack(wA[j], fa);
          Vec<T>::unpack(wB[j], fb);
          Vec<T>::unpack(xs[vv], xf);
#pragma unroll
          for (int e = 0; e < VW; e += 2) {
            a0 = fmaf(fa[e], xf[e], a0);
            a1 = fmaf(fa[e + 1], xf[e + 1], a1);
            b0 = fmaf(fb[e], xf[e], b0);
            b1 = fmaf(fb[e + 1], xf[e + 1], b1);
          }
        }
      }
    }
    const float sa = wave_sum(a0 + a1);
    const float sb = wave_sum(b0 + b1);
    if (lane == 0) {
      store_y<T>(cd, r, sa);
      if (two) store_y<T>(cd, r + kWaves, sb);
    }
  }
}

template <typename T, int UNROLL, int MODE>
__global__ void __launch_bounds__(kBlock) apply_kernel(KArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int n = a.n;
  const size_t pref_bytes = align_up((uint64_t)(n + 1) * 4, 16);
  const size_t g_bytes = align_up((uint64_t)a.max_k * 4, 16);
  int *pref = reinterpret_cast<int *>(smem);
  float *gs = reinterpret_cast<float *>(smem + pref_bytes);
  uint4 *xs = reinterpret_cast<uint4 *>(smem + pref_bytes + g_bytes);
  float *scr = reinterpret_cast<float *>(smem + pref_bytes + g_bytes +
                                         align_up((uint64_t)a.max_d * sizeof(T), 16));

  // Prefix over calls of the units their chosen path needs (written by the
  // projection launch).
  for (int i = tid; i <= n; i += kBlock) pref[i] = a.pref[i];
  __syncthreads();
  const int total = pref[n];

  // Each workgroup takes a contiguous range of units, so x or g is staged
  // again only when the range crosses into the next call.
  const int u0 = (int)((int64_t)total * blockIdx.x / gridDim.x);
  const int u1 = (int)((int64_t)total * (blockIdx.x + 1) / gridDim.x);
  int cur = -1;
  int c = 0;
  if (u0 < u1) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= u0)
        lo = mid;
      else
        hi = mid - 1;
    }
    c = lo;
  }
  CallDesc cd;
  bool slow = false;
  for (int u = u0; u < u1; ++u) {
    while (pref[c + 1] <= u) ++c;
    const int local = u - pref[c];
    if (c != cur) {
      cd = load_call(a, c);
      const float4 gi = reinterpret_cast<const float4 *>(a.gate)[cd.gate_off];
      slow = __float_as_int(gi.y) != 0;
      __syncthreads();
      if (slow) {
        const int nv = cd.d / Vec<T>::VW;
        const uint4 *xp = static_cast<const uint4 *>(cd.x);
        for (int i = tid; i < nv; i += kBlock) xs[i] = xp[i];
      } else {
        for (int j = tid; j < cd.k; j += kBlock) gs[j] = a.wsf[cd.g_off + j];
      }
      __syncthreads();
      cur = c;
    }
    if (slow)
      slow_unit<T, UNROLL>(cd, local, xs);
    else
      fast_unit<T, UNROLL>(cd, local, gs, scr);
  }
}

// ---------------------------------------------------------------------------
// Single-launch stack: projection, gate and output of every call of a plan
// in one persistent launch.
//
// Waves run one after the other.  Within wave w there are projection units
// (a fixed count) and output units (a count known per call once its gate is
// decided), both handed out as tickets (see take_ticket).  The workgroup that decides a call's gate
// opens it by appending the call to the wave's open list: one 64-bit
// fetch-add on the wave's open word (open calls << 40 | their output units)
// returns both the call's slot and the output ticket of its first unit, so
// output tickets number the units of the open calls in the order their
// gates opened.  Each workgroup holds one projection ticket and one output
// ticket of its wave.  It runs the output unit as soon as the open units
// cover its output ticket (finding the covering call by scanning the open
// list 64 slots at a time with the lanes of wavefront 0), otherwise a
// projection unit, and fetches the next ticket of the kind it used while the
// unit runs; once its group's output tickets are used up it takes them from
// the group with the most left before it leaves the wave.  No workgroup
// walks calls or polls a single call's word, which keeps the control traffic
// off any one memory channel.
//
// A workgroup waits only (a) when its wave has no projection ticket left and
// its output ticket is not covered yet: every gate it can wait for belongs
// to a call whose projection units are all held by running workgroups,
// which never wait inside the wave; or (b) on entering wave w+1, which it
// does only once wave w has no ticket left: every unit of wave w is then
// held by a running workgroup that waits on nothing later.  By induction
// over waves every wait ends, whatever the number of resident workgroups.
// Each wait is also bounded (spin_limit polls); if one ever runs out the
// workgroup sets the sticky status word and leaves, so the launch always
// drains.
//
// Within a wave, a call's output work starts as soon as its own gate opens,
// overlapping the projection of other calls, and no launch boundary
// separates the phases.
//
// Cross-workgroup data (partials, g, control words, and activations handed
// between waves) moves with agent-coherent accesses only, as in
// proj_kernel; s_waitcnt 0 before a barrier orders a workgroup's stores
// before the control word that publishes them.
// ---------------------------------------------------------------------------
enum { kJobDone = 0, kJobProj = 1, kJobOut = 2, kJobOutStatic = 3 };

// Latency-bound waves (at most kCdCache calls, each with one-tile fast
// units and its own projection) number their output tickets statically, in
// plan order: first every call's fast tiles (each ticket also the call's
// slow unit of the same index if its gate goes slow), then the slow units
// beyond those.  A workgroup holding such a ticket knows its call and unit
// before the gate is decided: it issues the loads of its image tile, then
// waits for the call's gate word (written by the finishing workgroup once
// g has landed), then needs only g.  The open list is not used there.
#ifndef GSI_STATIC_WAVES
#define GSI_STATIC_WAVES 1
#endif
// Polls of a gate word before the image tile's loads are issued (they are
// issued at once if the gate is decided earlier), and the sleep between
// polls (units of 64 clocks).
#ifndef GSI_STATIC_PREFETCH_DELAY
#define GSI_STATIC_PREFETCH_DELAY 0
#endif
#ifndef GSI_STATIC_POLL_SLEEP
#define GSI_STATIC_POLL_SLEEP 1
#endif

// Rows of V_k in flight per thread in a projection unit of the single-launch
// kernel.
#ifndef GSI_STACK_PROJ_UNROLL
#define GSI_STACK_PROJ_UNROLL 8
#endif

__device__ __forceinline__ uint32_t ctl_load(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ctl_load64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctl_add(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ctl_add64(uint64_t *p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_max(uint32_t *p, uint32_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_store(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_store64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The scheduler runs on the 64 lanes of wavefront 0.  Control words are
// touched by lane 0 only and broadcast; the open-list scan uses every lane.
__device__ __forceinline__ uint32_t bcast(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t bcast64(uint64_t v) {
  return ((uint64_t)bcast((uint32_t)(v >> 32)) << 32) | bcast((uint32_t)v);
}

constexpr uint64_t kLow40 = ((uint64_t)1 << 40) - 1;

// Scheduler state of one workgroup (uniform over wavefront 0; the tickets
// live in lane 0 between a fetch and their next use).
struct Sched {
  int w;          // current wave
  int entered;    // first tickets of wave w taken
  int p_out;      // projection tickets of wave w known exhausted
  int p_held;     // st.tp holds a projection ticket not yet run
  int last_out;   // the last job was an output unit
  int pf;         // ticket to fetch while the job runs: 1 projection, 2 output
  int slot;       // first open-list slot that may hold the output ticket
  uint32_t tp;    // projection ticket held
  uint32_t to;    // output ticket held
  uint64_t open;  // last open word seen for wave w
  int fresh;      // first pass after entering wave w
  int uc0;        // call of the first (static) projection ticket of wave w, or -1
  int stat;       // wave w numbers its output tickets statically (see kJobOutStatic)
  int vg;         // group whose counter hands out this workgroup's output tickets
};

// Descriptors of the calls of the current wave, copied to LDS when a
// workgroup enters the wave (while it waits for the previous wave), for
// waves of at most kCdCache calls: a latency-bound wave's jobs then read
// their call from LDS instead of making a round trip to the plan.
#ifndef GSI_CD_CACHE
#define GSI_CD_CACHE 1
#endif
constexpr int kCdCache = 4;
struct CdCache {
  CallDesc cd[kCdCache];
  int q0, n;  // first call of the wave and the count cached (0: none)
};

// Tickets of a wave: the first of each kind is the workgroup's index; the
// later ones of group g = blockIdx % kGroups are gridDim + kGroups * j + g
// for j = 0, 1, ... taken from group g's counter.  Every ticket from the
// grid size on belongs to exactly one group's counter, which hands it out
// once: the group's workgroups take its tickets in order until they pass
// the wave's count (and, at the end of a wave, workgroups of groups that
// have run out of output tickets).
__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr0, uint32_t g) {
  return gridDim.x + kGroups * ctl_add(ctr0 + 32 * g, 1u) + g;
}
__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr0) { return take_ticket(ctr0, blockIdx.x % kGroups); }

// The groups use up their output tickets at different times (their
// workgroups run units of different lengths), so a workgroup whose group
// has none left takes them from the group furthest behind before it leaves
// the wave (a ticket belongs to one group's counter, whoever takes it).
#ifndef GSI_STEAL_TAIL
#define GSI_STEAL_TAIL 1
#endif

// Lanes 0..7 read the groups' counters at ctr0; returns, uniform over the
// wavefront, (tickets below `total` left in the fullest group) << 3 | that
// group.  (Group tickets start at the grid size.)
__device__ __forceinline__ uint32_t fullest_group(uint32_t *ctr0, uint32_t total, int lane) {
  uint32_t key = (uint32_t)lane;
  if (lane < kGroups) {
    const uint32_t nt = gridDim.x + kGroups * ctl_load(ctr0 + 32 * lane) + (uint32_t)lane;
    key |= (nt < total ? (total - nt) : 0u) << 3;
  }
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) {
    const uint32_t other = (uint32_t)__shfl_xor((int)key, o, 64);
    key = other > key ? other : key;
  }
  return bcast(key);
}

__device__ __forceinline__ uint32_t *wave_ctl(const FArgs &a, int w) {
  return a.ctl + kCtlWave0 + w * kCtlWaveWords;
}

__device__ __forceinline__ void set_job(int *job, int kind, int c, int u, int slow) {
  if (threadIdx.x == 0) {
    job[0] = kind;
    job[1] = c;
    job[2] = u;
    job[3] = slow;
  }
}

__device__ __forceinline__ void sched_fail(const FArgs &a, int code, int *job) {
  if (threadIdx.x == 0) ctl_max(a.ctl + kCtlStatus, (uint32_t)code);
  set_job(job, kJobDone, 0, 0, 0);
}

__device__ __forceinline__ uint64_t load_open(const FArgs &a, int w) {
  uint64_t ow = 0;
  if (threadIdx.x == 0) ow = ctl_load64(reinterpret_cast<const uint64_t *>(wave_ctl(a, w) + kWvOpen));
  return bcast64(ow);
}

// Leave wave w.  The outputs this workgroup wrote in it have landed (each
// output unit of a wave with a successor ends with s_waitcnt 0 and a
// barrier).  The last workgroup of its group to leave counts the group; the
// last group raises the ready flags of the next wave's entry.
__device__ __forceinline__ void leave_wave(const FArgs &a, Sched &st, uint32_t *wv, int w, int lane) {
  if (lane == 0 && w + 1 < a.n_waves) {
    const uint32_t g = blockIdx.x % kGroups;
    const uint32_t gsize = (gridDim.x - g + kGroups - 1) / kGroups;
    if (ctl_add(wv + kWvLeft + 32 * g, 1u) == gsize - 1) {
      const uint32_t ngroups = gridDim.x < (uint32_t)kGroups ? gridDim.x : (uint32_t)kGroups;
      if (ctl_add(wv + kWvGroups, 1u) == ngroups - 1) {
#pragma unroll
        for (int q = 0; q < kGroups; ++q) ctl_store(wv + kWvReady + 32 * q, 1u);
      }
    }
  }
  st.w += 1;
  st.entered = 0;
}

// Picks the next job of this workgroup (wavefront 0): job = {kind, call,
// unit, slow} in LDS.  Within a wave a workgroup holds one output ticket
// and at most one projection ticket.  It runs its output unit as soon as
// the open units cover the ticket, otherwise a projection unit; a
// projection ticket fetched during a projection unit is run right after at
// most one output unit, so no ticket that gates other work is held for
// long.  It waits only when the wave has no projection ticket left, and
// leaves the wave once every gate is open and neither its output ticket nor
// any group's next one lies below the last unit.  The first ticket of each kind in a wave is the workgroup's
// own index (no atomic); the counters hand out the tickets from the grid
// size on.
__device__ void next_job(const FArgs &a, Sched &st, int *job, CdCache *cc) {
  const int lane = threadIdx.x;
  st.pf = 0;
  int polls = 0;
  for (;;) {
    if (st.w >= a.n_waves) break;
    const int w = st.w;
    uint32_t *wv = wave_ctl(a, w);
    if (!st.entered) {
      // what this wave's first jobs need from the plan, fetched before the
      // wait for the previous wave (plan data is never written in a launch)
      {
        const int p0e = a.wave_tab[w];
        const int npe = a.wave_tab[w + 1] - p0e;
        st.uc0 = (int)blockIdx.x < npe ? a.unit_call[p0e + blockIdx.x] : -1;
        const int q0e = a.wave_tab[a.n_waves + 1 + w];
        const int nqe = a.wave_tab[a.n_waves + 2 + w] - q0e;
        const int ncache = GSI_CD_CACHE && nqe <= kCdCache ? nqe : 0;
        constexpr int kWords = (int)(sizeof(CallDesc) / 4);
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.table + q0e);
        uint32_t *dst = reinterpret_cast<uint32_t *>(cc->cd);
        for (int i = lane; i < ncache * kWords; i += 64) dst[i] = src[i];
        if (lane == 0) {
          cc->q0 = q0e;
          cc->n = ncache;
        }
        int ok = 1;
        if (lane < ncache) {
          const CallDesc &dd = a.table[q0e + lane];
          ok = dd.fast_tiles == 1 && dd.share_next == 0 && dd.a_units > 0;
        }
        st.stat = GSI_STATIC_WAVES && ncache > 0 && ncache == nqe && __ballot(!ok) == 0;
      }
      if (w > 0) {
        // x of this wave may be y of the previous one: wait until every
        // workgroup has left that wave (each leaves once the wave has no
        // ticket for it, after its outputs landed; every unit of the wave is
        // held by a running workgroup).  The last one out raises a ready
        // flag on each group's own line, so that the pollers of one line
        // are a group, not the grid.
        const uint32_t *pv = wave_ctl(a, w - 1);
        for (int s = 0;; ++s) {
          uint32_t ok = 0;
          if (lane == 0) ok = ctl_load(pv + kWvReady + 32 * (blockIdx.x % kGroups));
          if (bcast(ok)) break;
          if (s >= a.spin_limit) return sched_fail(a, 1, job);
          __builtin_amdgcn_s_sleep(8);
        }
      }
      st.to = blockIdx.x;
      st.tp = blockIdx.x;
      st.vg = (int)(blockIdx.x % kGroups);
      st.entered = 1;
      st.p_out = 0;
      st.p_held = 1;
      st.last_out = 0;
      st.slot = 0;
      st.open = 0;
      st.fresh = 1;
    }
    const int p0 = a.wave_tab[w];
    const int np = a.wave_tab[w + 1] - p0;
    if (st.stat) {
      // every projection ticket before any output ticket: an output job
      // waits for its call's gate, which needs every projection unit
      if (!st.p_out) {
        if (!st.p_held) {
          uint32_t t = 0;
          if (lane == 0) t = take_ticket(wv + kWvProj);
          st.tp = t;
        }
        const uint32_t tp = bcast(st.tp);
        st.p_held = 0;
        if ((int)tp < np) {
          set_job(job, kJobProj, tp == blockIdx.x && st.uc0 >= 0 ? st.uc0 : a.unit_call[p0 + tp], p0 + (int)tp, 0);
          st.last_out = 0;
          st.pf = 1;
          return;
        }
        st.p_out = 1;
      }
      // output ticket -> (call, region, unit) from the cached descriptors
      const uint32_t to = bcast(st.to);
      uint32_t base = 0;
      for (int r = 0; r < 2; ++r)
        for (int i = 0; i < cc->n; ++i) {
          const int fu = cc->cd[i].fast_units, su = cc->cd[i].slow_units;
          const uint32_t cnt = (uint32_t)(r == 0 ? fu : (su > fu ? su - fu : 0));
          if (to - base < cnt) {
            set_job(job, kJobOutStatic, cc->q0 + i, (int)(to - base), r);
            st.last_out = 1;
            st.pf = 2;
            return;
          }
          base += cnt;
        }
      leave_wave(a, st, wv, w, lane);
      continue;
    }
    if (st.p_held && st.last_out) {
      // a projection ticket waited through one output unit: run it now
      const uint32_t tp = bcast(st.tp);
      st.p_held = 0;
      if ((int)tp < np) {
        set_job(job, kJobProj, tp == blockIdx.x && st.uc0 >= 0 ? st.uc0 : a.unit_call[p0 + tp], p0 + (int)tp, 0);
        st.last_out = 0;
        st.pf = 1;
        return;
      }
      st.p_out = 1;
    }
    const uint32_t to = bcast(st.to);
    const int q0 = a.wave_tab[a.n_waves + 1 + w];
    const uint32_t ncalls = (uint32_t)(a.wave_tab[a.n_waves + 2 + w] - q0);
    // (once every gate of the wave is open the cached open word is final;
    // the first pass after entering the wave skips the reload: gates open
    // only as projection units finish, so a workgroup that has just entered
    // runs its projection ticket first, and one without a ticket reloads on
    // its next pass)
    const int fresh = st.fresh;
    st.fresh = 0;
    if (!fresh && to >= (uint32_t)(st.open & kLow40) && (uint32_t)(st.open >> 40) != ncalls)
      st.open = load_open(a, w);
    if (to < (uint32_t)(st.open & kLow40)) {
      // ---- output unit: find the open call that covers ticket `to` ----
      const int nopen = (int)(st.open >> 40);
      for (int base_slot = st.slot;; base_slot += 64) {
        const int idx = base_slot + lane;
        uint64_t e = 0;
        int stuck = 0;
        if (idx < nopen) {
          e = ctl_load64(a.entries + q0 + idx);
          for (int s = 0; e == 0; ++s) {  // opened a moment ago, entry not yet stored
            if (s >= a.spin_limit) {
              stuck = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            e = ctl_load64(a.entries + q0 + idx);
          }
        }
        if (__ballot(stuck)) return sched_fail(a, 3, job);
        const uint32_t eb = (uint32_t)e;
        const uint32_t en = (uint32_t)(e >> 32) & ((1u << kEntryNeedBits) - 1);
        const uint64_t hit = __ballot(idx < nopen && to >= eb && to - eb < en);
        if (hit) {
          const int l = __ffsll((unsigned long long)hit) - 1;
          const uint64_t he =
              ((uint64_t)(uint32_t)__shfl((int)(e >> 32), l, 64) << 32) | (uint32_t)__shfl((int)eb, l, 64);
          st.slot = base_slot + l;
          set_job(job, kJobOut, (int)(he >> 51) - 1, (int)(to - (uint32_t)he), (int)((he >> 50) & 1));
          st.last_out = 1;
          st.pf = 2;
          return;
        }
        if (base_slot + 64 >= nopen) return sched_fail(a, 4, job);  // cannot happen: to < open units
      }
    }
    if ((uint32_t)(st.open >> 40) == ncalls && !(st.p_held && (int)bcast(st.tp) < np)) {
      // every gate of the wave is open, so every projection unit is done
      // and no projection ticket need be taken
      st.p_out = 1;
      st.p_held = 0;
    }
    if (!st.p_out) {
      // ---- projection unit ----
      if (!st.p_held) {
        uint32_t t = 0;
        if (lane == 0) t = take_ticket(wv + kWvProj);
        st.tp = t;
      }
      const uint32_t tp = bcast(st.tp);
      st.p_held = 0;
      if ((int)tp < np) {
        set_job(job, kJobProj, tp == blockIdx.x && st.uc0 >= 0 ? st.uc0 : a.unit_call[p0 + tp], p0 + (int)tp, 0);
        st.last_out = 0;
        st.pf = 1;
        return;
      }
      st.p_out = 1;
    }
    if ((uint32_t)(st.open >> 40) == ncalls) {  // every gate open and `to` beyond the last unit
      const uint32_t total = (uint32_t)(st.open & kLow40);
      if (GSI_STEAL_TAIL && total > gridDim.x) {
        // take a ticket from the group with the most left.  Each attempt
        // either gets a unit or finds that group exhausted, so the
        // workgroup leaves after at most kGroups empty attempts.
        const uint32_t key = fullest_group(wv + kWvOut, total, lane);
        if (key >> 3) {
          const uint32_t vg = key & 7u;
          uint32_t t = 0;
          if (lane == 0) t = take_ticket(wv + kWvOut, vg);
          st.to = t;
          st.vg = (int)vg;
          st.slot = 0;  // a ticket of another group may lie before the last one held
          continue;
        }
      }
      leave_wave(a, st, wv, w, lane);
      continue;
    }
    // nothing to do until another gate of this wave opens
    if (++polls > a.spin_limit) return sched_fail(a, 2, job);
    __builtin_amdgcn_s_sleep(8);
  }
  set_job(job, kJobDone, 0, 0, 0);
}

// Fetches the ticket of the kind the job used up (wavefront 0, right after
// the job was handed out; lane 0 takes the ticket, which the next call of
// next_job reads; the state flags stay uniform over the wavefront).
__device__ __forceinline__ void sched_prefetch(const FArgs &a, Sched &st) {
  if (st.pf == 1) {
    if (threadIdx.x == 0) st.tp = take_ticket(wave_ctl(a, st.w) + kWvProj);
    st.p_held = 1;
  } else if (st.pf == 2) {
    if (threadIdx.x == 0) st.to = take_ticket(wave_ctl(a, st.w) + kWvOut, (uint32_t)st.vg);
  }
}

// x of a call staged in LDS for its slow units (agent-coherent loads when
// an earlier wave of the launch wrote it).
template <typename T>
__device__ __forceinline__ void stage_x(const CallDesc &cd, uint4 *xs) {
  constexpr int VW = Vec<T>::VW;
  const int nv = cd.d / VW;
  if (cd.flags & kCallXCoherent) {
    const uint32_t *xw = static_cast<const uint32_t *>(cd.x);
    for (int i = threadIdx.x; i < nv; i += kBlock)
      xs[i] = make_uint4(ctl_load(xw + 4 * i), ctl_load(xw + 4 * i + 1), ctl_load(xw + 4 * i + 2),
                         ctl_load(xw + 4 * i + 3));
  } else {
    const uint4 *xp = static_cast<const uint4 *>(cd.x);
    for (int i = threadIdx.x; i < nv; i += kBlock) xs[i] = xp[i];
  }
}

// One static output ticket (see kJobOutStatic) of call c: region 0 = fast
// tile u or slow unit u, region 1 = slow unit fast_units + u.  Issues the
// tile's first loads, waits (bounded) for the call's gate word, then runs
// the unit the gate selects, if any.  Returns the path run (0 fast, 1 slow)
// or -1 for a void ticket.  cur / cur_slow: what xs / gs hold.
template <typename T, int UNROLL>
__device__ __forceinline__ int static_output(const FArgs &a, const CallDesc &cd, int c, int u, int region,
                                             int &cur, int &cur_slow, uint4 *xs, float *gs, float *scr,
                                             int *flag) {
  uint4 mv[UNROLL];
  if (region == 0 && GSI_STATIC_PREFETCH_DELAY < 0) fast_tile_load<T, UNROLL>(cd, u, mv);
  int gate = 0;
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) {
      uint64_t e = ctl_load64(a.entries + c);
      if (e == 0 && it >= a.spin_limit) {
        ctl_max(a.ctl + kCtlStatus, 5u);
        e = 3;
      }
      *flag = (int)e;
    }
    __syncthreads();
    gate = *flag;
    __syncthreads();
    if (GSI_STATIC_PREFETCH_DELAY >= 0 && region == 0 && (gate != 0 || it == GSI_STATIC_PREFETCH_DELAY) &&
        it <= GSI_STATIC_PREFETCH_DELAY)
      fast_tile_load<T, UNROLL>(cd, u, mv);
    if (gate) break;
    __builtin_amdgcn_s_sleep(GSI_STATIC_POLL_SLEEP);
  }
  if (gate == 1 && region == 0) {
    if (c != cur || cur_slow) {
      for (int j = threadIdx.x; j < cd.k; j += kBlock) gs[j] = load_coherent(a.wsf + cd.g_off + j);
      __syncthreads();
      cur = c;
      cur_slow = 0;
    }
    fast_tile_finish<T, UNROLL>(cd, u, mv, gs, scr);
    return 0;
  }
  const int su = region == 0 ? u : cd.fast_units + u;
  if (gate == 2 && su < cd.slow_units) {
    if (c != cur || !cur_slow) {
      stage_x<T>(cd, xs);
      __syncthreads();
      cur = c;
      cur_slow = 1;
    }
    slow_unit<T, UNROLL>(cd, su, xs);
    return 1;
  }
  return -1;
}

// Two workgroups of four wavefronts per CU (see launch_stack_mode): the
// register budget of two wavefronts per SIMD lets the compiler keep every
// streaming load of a unit in flight (measured 290 -> 238 us per 112-map
// step against the default budget).
#ifndef GSI_STACK_WAVES_PER_EU
#define GSI_STACK_WAVES_PER_EU 2
#endif
#define GSI_STACK_ATTR __attribute__((amdgpu_waves_per_eu(1, GSI_STACK_WAVES_PER_EU)))

template <typename T, int UNROLL, int MODE>
__global__ void __launch_bounds__(kBlock) GSI_STACK_ATTR stack_kernel(FArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float sh[kWaves];
  __shared__ int s_job[4];
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  // Output units use x (slow) or g (fast) staged at the start of the LDS
  // block; projection units use it for their column partials.
  uint4 *xs = reinterpret_cast<uint4 *>(smem);
  float *gs = reinterpret_cast<float *>(smem + align_up((uint64_t)a.max_d * sizeof(T), 16));
  float *scr = gs + align_up((uint64_t)a.max_k, 4);
  float *red = reinterpret_cast<float *>(smem);

  Sched st{0, 0, 0, 0, 0, 0, 0, 0u, 0u, 0, 0, -1, 0, 0};
  __shared__ __align__(16) CdCache cc;
  int cur = -1, cur_slow = 0;
  GSI_TRACE_ONLY(unsigned tn = 0; unsigned long long tj = wall_clock64(); if (tid == 0) trace_rec(tn, tj, tj, 9, 0, 0, 0);)
  for (;;) {
    GSI_TRACE_ONLY(const unsigned long long tq = wall_clock64();)
    if (tid < 64) next_job(a, st, s_job, &cc);
    __syncthreads();
    const int kind = s_job[0];
    const int c = __builtin_amdgcn_readfirstlane(s_job[1]);
    const int u = s_job[2];
    const int slow = s_job[3];
    __syncthreads();  // s_job is rewritten only after every thread has read it
    GSI_TRACE_ONLY(tj = wall_clock64(); if (tid == 0) trace_rec(tn, tq, tj, 8, 0, 0, 0);)
    if (kind == kJobDone) break;
    if (tid < 64) sched_prefetch(a, st);
    const int ci = c - cc.q0;
    const CallDesc cd = ci >= 0 && ci < cc.n ? cc.cd[ci] : a.table[c];
    GSI_TRACE_ONLY(int t_kind = kind; int t_u = u; int t_slow = slow;)
    if (kind == kJobProj) {
      cur = -1;  // the partials overwrite staged x / g
      const int q = u - cd.a_begin;
      float *part = a.wsf + cd.part_off + (int64_t)q * (cd.k + 4);
      if (cd.flags & kCallXCoherent)
        proj_partial<T, GSI_STACK_PROJ_UNROLL, true>(cd, q, part, red, sh);
      else
        proj_partial<T, GSI_STACK_PROJ_UNROLL, false>(cd, q, part, red, sh);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (projection_handoff(cd, c, q, a.wsf, a.counters, a.gcounters, &s_flag)) {
        int rows = 0;
        const float *p0 = final_rows(cd, a.wsf, &rows);
        const float3 r = finish_projection<T, true>(cd, p0, rows, a.wsf + cd.g_off, a.counters, sh, red);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // g of every thread is stored before any gate opens
        if (tid == 0 && st.stat) {
          // a wave with static output tickets: publish the gate in the call's word
          const int sl = decide_gate<MODE>(cd, r, a.gate);
          ctl_store64(a.entries + c, 1u + (uint64_t)sl);
        } else if (tid == 0) {
          // open the gates of this call and of every call sharing its
          // projection: append each to its wave's open list
          uint32_t *wv = wave_ctl(a, cd.wave);
          for (int m = c;;) {
            const CallDesc md = m == c ? cd : a.table[m];
            const int sl = decide_gate<MODE>(md, r, a.gate);
            const uint64_t need = (uint64_t)(sl ? md.slow_units : md.fast_units);
            const uint64_t old = ctl_add64(reinterpret_cast<uint64_t *>(wv + kWvOpen), ((uint64_t)1 << 40) | need);
            ctl_store64(a.entries + a.wave_tab[a.n_waves + 1 + md.wave] + (old >> 40),
                        (old & kLow40) | (need << 32) | ((uint64_t)sl << 50) | ((uint64_t)(m + 1) << 51));
            if (md.share_next == 0) break;
            m = md.share_next - 1;
          }
        }
      }
    } else if (kind == kJobOutStatic) {
      // A static output ticket: region `slow` of the call's tickets, 0 = fast
      // tile u (or slow unit u), 1 = slow unit fast_units + u.  The tile's
      // first loads go out before the wait for the gate.
      const int sl = static_output<T, UNROLL>(a, cd, c, u, slow, cur, cur_slow, xs, gs, scr, &s_flag);
      GSI_TRACE_ONLY(t_kind = sl >= 0 ? kJobOut : 10; t_slow = sl; t_u = slow && sl > 0 ? cd.fast_units + u : u;)
      (void)sl;
      if (cd.wave + 1 < a.n_waves) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    } else {
      if (c != cur || slow != cur_slow) {
        if (slow)
          stage_x<T>(cd, xs);
        else
          for (int j = tid; j < cd.k; j += kBlock) gs[j] = load_coherent(a.wsf + cd.g_off + j);
        __syncthreads();
        cur = c;
        cur_slow = slow;
      }
      if (slow)
        slow_unit<T, UNROLL>(cd, u, xs);
      else
        fast_unit<T, UNROLL>(cd, u, gs, scr);
      if (cd.wave + 1 < a.n_waves) {
        // a later wave may read this y: its stores land before the
        // workgroup can leave the wave
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
    GSI_TRACE_ONLY(__builtin_amdgcn_s_waitcnt(0); if (tid == 0) trace_rec(tn, tj, wall_clock64(), t_kind, c, t_u, t_slow);)
  }
  GSI_TRACE_ONLY(if (tid == 0) { const unsigned long long te = wall_clock64(); trace_rec(tn, te, te, 7, 0, 0, 0); })

  // The last workgroup to leave clears the control words (all but the status
  // word) and the projection counters for the next launch on this workspace;
  // also the group counters of two-level sums, which a completed launch has
  // already cleared, but a launch whose wait bound ran out may have left
  // counting a group whose units did not all run.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_flag = ctl_add(a.ctl + kCtlExit, 1u) == gridDim.x - 1 ? 1 : 0;
  __syncthreads();
  if (!s_flag) return;
  for (int i = tid; i < a.n_waves * kCtlWaveWords; i += kBlock) ctl_store(a.ctl + kCtlWave0 + i, 0u);
  for (int i = tid; i < a.n; i += kBlock) {
    ctl_store64(a.entries + i, 0u);
    ctl_store(a.counters + i, 0u);
  }
  for (int i = tid; i < a.units_a; i += kBlock) ctl_store(a.gcounters + i, 0u);
  if (tid == 0) {
    ctl_store(a.ctl + kCtlSeg, 0u);
    ctl_store(a.ctl + kCtlExit, 0u);
  }
}

// ---------------------------------------------------------------------------
// M = W V_k into the tiled layout (one 64-row tile x up to 256 columns per
// workgroup; fp32 FMA over d in chunks of 32 staged through LDS).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kBlock)
    prepare_kernel(const T *__restrict__ W, const T *__restrict__ V, T *__restrict__ M, int d,
                   int d_out, int k) {
  constexpr int VW = Vec<T>::VW;
  constexpr int KC = 32;
  __shared__ float Ws[kTileRows][KC + 1];
  __shared__ float Vs[KC][256];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int cb = blockIdx.y * 256;
  const int r = tid & 63;
  const int cgi = tid >> 6;  // 64-column group of this thread
  float acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += KC) {
    for (int i = tid; i < kTileRows * KC; i += kBlock) {
      const int rr = i / KC, cc = i % KC;
      const int gr = tile * kTileRows + rr, gc = k0 + cc;
      Ws[rr][cc] = (gr < d_out && gc < d) ? Vec<T>::load1(W, (size_t)gr * d + gc) : 0.f;
    }
    for (int i = tid; i < KC * 256; i += kBlock) {
      const int rr = i / 256, cc = i % 256;
      const int gr = k0 + rr, gc = cb + cc;
      Vs[rr][cc] = (gr < d && gc < k) ? Vec<T>::load1(V, (size_t)gr * k + gc) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      const float w = Ws[r][kk];
#pragma unroll
      for (int j = 0; j < 64; ++j) acc[j] = fmaf(w, Vs[kk][cgi * 64 + j], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const int c = cb + cgi * 64 + j;
    if (c < k) {
      const size_t idx = (size_t)tile * kTileRows * k + (size_t)(c / VW) * kTileRows * VW +
                         (size_t)r * VW + (c % VW);
      Vec<T>::store1(M, idx, acc[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// E = V_k^T V_k - I (k x k, row-major, storage dtype) for the exact residual
// ratio: one 64 x 64 block of E per workgroup, fp64 FMA over the d rows of
// V_k in chunks of 32 staged through LDS (the diagonal sums d squares to
// nearly 1 before 1 is subtracted, which fp32 would leave ~4e-6 off).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kBlock) gram_kernel(const T *__restrict__ V, T *__restrict__ E, int d, int k) {
  constexpr int KC = 32;
  __shared__ float Vi[KC][64];
  __shared__ float Vj[KC][65];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int ri = tid >> 2;          // row of the block (0..63)
  const int cj = (tid & 3) * 16;    // first of 16 columns
  double acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = 0.0;
  for (int r0 = 0; r0 < d; r0 += KC) {
    for (int e = tid; e < KC * 64; e += kBlock) {
      const int r = e / 64, c = e % 64;
      const bool ok = r0 + r < d;
      Vi[r][c] = (ok && i0 + c < k) ? Vec<T>::load1(V, (size_t)(r0 + r) * k + i0 + c) : 0.f;
      Vj[r][c] = (ok && j0 + c < k) ? Vec<T>::load1(V, (size_t)(r0 + r) * k + j0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < KC; ++r) {
      const double a = Vi[r][ri];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = fma(a, (double)Vj[r][cj + c], acc[c]);
    }
    __syncthreads();
  }
  const int i = i0 + ri;
  if (i < k) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int j = j0 + cj + c;
      if (j < k) Vec<T>::store1(E, (size_t)i * k + j, (float)(acc[c] - (i == j ? 1.0 : 0.0)));
    }
  }
}

hipError_t launch_gram(int dtype, const void *V, void *E, int d, int k, hipStream_t s) {
  const dim3 grid((k + 63) / 64, (k + 63) / 64);
  if (dtype == 0)
    hipLaunchKernelGGL(gram_kernel<float>, grid, dim3(kBlock), 0, s, static_cast<const float *>(V),
                       static_cast<float *>(E), d, k);
  else
    hipLaunchKernelGGL(gram_kernel<bf16_t>, grid, dim3(kBlock), 0, s, static_cast<const bf16_t *>(V),
                       static_cast<bf16_t *>(E), d, k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from gsi_api.cpp).
// ---------------------------------------------------------------------------
hipError_t launch_prepare_bf16(const void *W, const void *V, void *M, int d, int d_out, int k,
                               hipStream_t s);

// bf16 images are built on the matrix cores (gsi_batched.hip); fp32 images
// with the FMA kernel above.
hipError_t launch_prepare(int dtype, const void *W, const void *V, void *M, int d, int d_out,
                          int k, hipStream_t s) {
  if (dtype != 0) return launch_prepare_bf16(W, V, M, d, d_out, k, s);
  const dim3 grid((d_out + kTileRows - 1) / kTileRows, (k + 255) / 256);
  hipLaunchKernelGGL(prepare_kernel<float>, grid, dim3(kBlock), 0, s,
                     static_cast<const float *>(W), static_cast<const float *>(V),
                     static_cast<float *>(M), d, d_out, k);
  return hipGetLastError();
}

size_t apply_lds_bytes(const KArgs &a, int esize) {
  return align_up((uint64_t)(a.n + 1) * 4, 16) + align_up((uint64_t)a.max_k * 4, 16) +
         align_up((uint64_t)a.max_d * esize, 16) + kWaves * 64 * 4;
}

#ifndef GSI_PROJ_UNROLL
#define GSI_PROJ_UNROLL 8
#endif

template <typename T, int MODE>
void launch_modes(const KArgs &a, int grid_b, int phases, size_t lds, hipStream_t s) {
  constexpr int U = 8;
  constexpr int UP = GSI_PROJ_UNROLL;
  if (phases & 1)
    hipLaunchKernelGGL((proj_kernel<T, UP, MODE>), dim3(a.units_a), dim3(kBlock), 0, s, a);
  if (phases & 2)
    hipLaunchKernelGGL((apply_kernel<T, U, MODE>), dim3(grid_b), dim3(kBlock), lds, s, a);
}

template <typename T>
void launch_typed(const KArgs &a, int grid_b, int phases, size_t lds, hipStream_t s) {
  if (a.mode == 1)
    launch_modes<T, 1>(a, grid_b, phases, lds, s);
  else if (a.mode == 2)
    launch_modes<T, 2>(a, grid_b, phases, lds, s);
  else
    launch_modes<T, 0>(a, grid_b, phases, lds, s);
}

size_t stack_lds_bytes(int max_d, int max_k, int esize) {
  const size_t out = align_up((uint64_t)max_d * esize, 16) + align_up((uint64_t)max_k * 4, 16) +
                     kWaves * 64 * 4;
  const size_t proj = (size_t)kBlock * (16 / esize) * 4;
  return out > proj ? out : proj;
}

#ifndef GSI_STACK_GROUPS_PER_CU
#define GSI_STACK_GROUPS_PER_CU 2
#endif
constexpr size_t kLdsPerCu = 160 * 1024;

#ifndef GSI_STACK_UNROLL
#define GSI_STACK_UNROLL 8
#endif

template <typename T, int MODE>
hipError_t launch_stack_mode(const FArgs &a, int max_groups, hipStream_t s) {
  constexpr int U = GSI_STACK_UNROLL;
  // Fewer concurrent streams than the registers allow read HBM faster
  // (512 workgroups beat 768 on the 112-map step), and they must be spread
  // evenly over the CUs: the LDS request is raised so that at most
  // GSI_STACK_GROUPS_PER_CU workgroups fit on one CU.
  size_t lds = stack_lds_bytes(a.max_d, a.max_k, (int)sizeof(T));
  const size_t spread = kLdsPerCu / (GSI_STACK_GROUPS_PER_CU + 1) + 1024;
  if (lds < spread && spread * GSI_STACK_GROUPS_PER_CU <= kLdsPerCu) lds = spread;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, stack_kernel<T, U, MODE>, kBlock, lds) !=
          hipSuccess || occ < 1)
    occ = 1;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  int grid = occ * cus;
  if (max_groups > 0 && grid > max_groups) grid = max_groups;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((stack_kernel<T, U, MODE>), dim3(grid), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_stack_typed(const FArgs &a, int mode, int max_groups, hipStream_t s) {
  if (mode == 1) return launch_stack_mode<T, 1>(a, max_groups, s);
  if (mode == 2) return launch_stack_mode<T, 2>(a, max_groups, s);
  return launch_stack_mode<T, 0>(a, max_groups, s);
}

hipError_t launch_stack(int dtype, const FArgs &a, int mode, int max_groups, hipStream_t s) {
  if (dtype == 0) return launch_stack_typed<float>(a, mode, max_groups, s);
  return launch_stack_typed<bf16_t>(a, mode, max_groups, s);
}

hipError_t launch_batch1(int dtype, const KArgs &a, int grid_b, int phases, hipStream_t s) {
  const int esize = dtype == 0 ? 4 : 2;
  const size_t lds = apply_lds_bytes(a, esize);
  if (dtype == 0)
    launch_typed<float>(a, grid_b, phases, lds, s);
  else
    launch_typed<bf16_t>(a, grid_b, phases, lds, s);
  return hipGetLastError();
}

}  // namespace gsi

#if GSI_TRACE
// Copies the record slots (4 x uint64 each; zero = unused), at most
// max_entries of them, to host memory; returns the count copied, or a
// negative value on a HIP error.
extern "C" int gsi_trace_read(unsigned long long *host, int max_entries) {
  size_t n = (size_t)gsi::kTraceBlocks * gsi::kTracePer;
  if (max_entries < 0) max_entries = 0;
  if (n > (size_t)max_entries) n = (size_t)max_entries;
  if (n && hipMemcpyFromSymbol(host, HIP_SYMBOL(gsi::g_trace), n * 32) != hipSuccess) return -2;
  return (int)n;
}

// Zeroes every slot (synchronous).
extern "C" int gsi_trace_reset(void) {
  void *p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(gsi::g_trace)) != hipSuccess || !p) return -1;
  if (hipMemset(p, 0, sizeof(gsi::g_trace)) != hipSuccess) return -1;
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}
#endif
