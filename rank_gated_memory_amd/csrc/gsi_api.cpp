// C ABI of libgsi: argument checks, workspace sizing, stack plans, launches.
// The operations themselves are defined in include/gsi.h and follow the
// technical summary of "Gated Subspace Inference for Transformer
// Acceleration" (S. J. Thomas, 2026), §2.1-§2.2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/gsi.h"
#include "gsi_batched.h"
#include "gsi_calib.h"
#include "gsi_internal.h"

namespace gsi {
hipError_t launch_prepare(int dtype, const void *W, const void *V, void *M, int d, int d_out,
                          int k, hipStream_t s);
hipError_t launch_batch1(int dtype, const KArgs &a, int grid_b, int phases, hipStream_t s);
hipError_t launch_stack(int dtype, const FArgs &a, int mode, int max_groups, hipStream_t s);
hipError_t launch_gram(int dtype, const void *V, void *E, int d, int k, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs &c, hipStream_t s);
hipError_t launch_batched(const BArgs &a, hipStream_t s);
}  // namespace gsi

using namespace gsi;

namespace {

int esize_of(int32_t dtype) { return dtype == GSI_FP32 ? 4 : (dtype == GSI_BF16 ? 2 : 0); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gsi_status check_shape(int32_t d, int32_t d_out, int32_t k, int32_t dtype) {
  const int es = esize_of(dtype);
  if (es == 0) return GSI_E_DTYPE;
  if (d <= 0 || d_out <= 0 || k <= 0) return GSI_E_SHAPE;
  if (d % 8 || d_out % 8 || k % 8) return GSI_E_SHAPE;
  if (k > d || k > kMaxK) return GSI_E_SHAPE;
  if ((int64_t)d * es > kMaxRowBytes) return GSI_E_SHAPE;
  return GSI_OK;
}

gsi_status check_map(const gsi_map *m) {
  if (!m) return GSI_E_NULL;
  const gsi_status s = check_shape(m->d, m->d_out, m->k, m->dtype);
  if (s != GSI_OK) return s;
  if (!m->W || !m->V || !m->M) return GSI_E_NULL;
  if (!aligned(m->W, 16) || !aligned(m->V, 16) || !aligned(m->M, 16) || !aligned(m->G, 16))
    return GSI_E_ALIGN;
  return GSI_OK;
}

// Device compute-unit count (cached per device); sizes the persistent grid.
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

#ifndef GSI_APPLY_BLOCKS_PER_CU
#define GSI_APPLY_BLOCKS_PER_CU 32
#endif

struct WsLayout {
  uint64_t gate_off, need_off, pref_off, float_off, ctl_off, gcnt_off, total;
};

// The group counters of two-level partial sums follow the control words.
uint64_t gcnt_offset(uint64_t ctl_off, int64_t ctl) { return align_up(ctl_off + (uint64_t)ctl * 4, 256); }

// ctl: control words of the single-launch stack kernel (0 for gsi_linear);
// units_a: projection units (at most one group counter each)
WsLayout ws_layout(int64_t n, int64_t floats, int64_t ctl, int64_t units_a) {
  WsLayout w;
  w.gate_off = align_up((uint64_t)(n + 1) * 4, 256);
  w.need_off = align_up(w.gate_off + (uint64_t)n * 16, 256);
  w.pref_off = align_up(w.need_off + (uint64_t)n * 4, 256);
  w.float_off = align_up(w.pref_off + (uint64_t)(n + 1) * 4, 256);
  w.ctl_off = align_up(w.float_off + (uint64_t)floats * 4, 256);
  w.gcnt_off = gcnt_offset(w.ctl_off, ctl);
  w.total = align_up(w.gcnt_off + (uint64_t)units_a * 4, 256);
  return w;
}

void set_ws(KArgs &a, void *ws, uint64_t gate_off, uint64_t need_off, uint64_t pref_off,
            uint64_t float_off, uint64_t gcnt_off) {
  char *b = static_cast<char *>(ws);
  a.counters = reinterpret_cast<uint32_t *>(b);
  a.gcounters = reinterpret_cast<uint32_t *>(b + gcnt_off);
  a.gate = b + gate_off;
  a.need = reinterpret_cast<int32_t *>(b + need_off);
  a.pref = reinterpret_cast<int32_t *>(b + pref_off);
  a.wsf = reinterpret_cast<float *>(b + float_off);
}

int apply_grid(int64_t units_b_max) {
  int64_t g = (int64_t)cu_count() * GSI_APPLY_BLOCKS_PER_CU;
  if (units_b_max < g) g = units_b_max;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

int32_t gsi_abi_version(void) { return GSI_ABI_VERSION; }

const char *gsi_status_str(int32_t s) {
  switch (s) {
    case GSI_OK: return "GSI_OK";
    case GSI_E_NULL: return "GSI_E_NULL";
    case GSI_E_SHAPE: return "GSI_E_SHAPE";
    case GSI_E_DTYPE: return "GSI_E_DTYPE";
    case GSI_E_ALIGN: return "GSI_E_ALIGN";
    case GSI_E_WORKSPACE: return "GSI_E_WORKSPACE";
    case GSI_E_HIP: return "GSI_E_HIP";
    case GSI_E_ARG: return "GSI_E_ARG";
    default: return "GSI_E_UNKNOWN";
  }
}

size_t gsi_image_bytes(int32_t d_out, int32_t k, int32_t dtype) {
  const int es = esize_of(dtype);
  if (es == 0 || d_out <= 0 || k <= 0) return 0;
  const int64_t tiles = (d_out + kTileRows - 1) / kTileRows;
  return (size_t)(tiles * kTileRows * (int64_t)k * es);
}

size_t gsi_gram_bytes(int32_t k, int32_t dtype) {
  const int es = esize_of(dtype);
  if (es == 0 || k <= 0) return 0;
  return (size_t)k * k * es;
}

gsi_status gsi_prepare(const gsi_map *map, void *stream) {
  const gsi_status s = check_map(map);
  if (s != GSI_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_prepare(map->dtype, map->W, map->V, map->M, map->d, map->d_out, map->k, st);
  if (e == hipSuccess && map->G) e = launch_gram(map->dtype, map->V, map->G, map->d, map->k, st);
  return e == hipSuccess ? GSI_OK : GSI_E_HIP;
}

// Bytes of V_k per projection unit of a stack plan: small enough that the
// gates of a step open progressively (output work overlaps projection in
// the single launch), large enough to amortise a unit's partial hand-off.
#ifndef GSI_PLAN_PROJ_UNIT_KB
#define GSI_PLAN_PROJ_UNIT_KB 384
#endif
static int64_t plan_proj_target(int64_t total_v_bytes) {
  int64_t t = total_v_bytes / (256 * 4);
  if (t < 16 * 1024) t = 16 * 1024;
  if (t > GSI_PLAN_PROJ_UNIT_KB * 1024) t = GSI_PLAN_PROJ_UNIT_KB * 1024;
  return t;
}

// Unit shapes of every call of a (validated) plan, chosen wave by wave.
// A wave's projection units aim at (its V_k bytes) / 1024, clamped to
// [16 KiB, GSI_PLAN_PROJ_UNIT_KB], and at most kMaxPartials per call (the
// final sum of a call's partials is then one round of loads).  A wave whose fast
// outputs make fewer than kFineUnits ordinary units is latency-bound (the
// waves of a dependency-chained stack): it takes the smallest output units.
constexpr int64_t kFineUnits = 1024;
#ifndef GSI_PLAN_MAX_PARTIALS
#define GSI_PLAN_MAX_PARTIALS 64
#endif
constexpr int64_t kMaxPartials = GSI_PLAN_MAX_PARTIALS;
constexpr int64_t kTwoLevelUnitBytes = 64 * 1024;
constexpr int64_t kMaxPartials2 = 256;

// Unit shape of one call in a wave whose projection bytes total `wave_vbytes`
// and whose fast outputs make `wave_fast_units` ordinary units (the rule
// above).
static UnitShape shape_in_wave(int32_t d, int32_t d_out, int32_t k, int es, int64_t wave_vbytes,
                               int64_t wave_fast_units) {
  const int64_t t = plan_proj_target(wave_vbytes);
  const bool fine = wave_fast_units < kFineUnits;
  const int64_t vi = (int64_t)d * k * es;
  int64_t ti = std::max<int64_t>(t, (vi + kMaxPartials - 1) / kMaxPartials);
  // Where the cap of kMaxPartials one-level partials would make the units
  // larger than the wave's target and than kTwoLevelUnitBytes (a wide V_k in
  // a latency-bound wave), up to kMaxPartials2 smaller units are summed in
  // two levels instead.
  if (ti > t && ti > kTwoLevelUnitBytes)
    ti = std::max<int64_t>({t, kTwoLevelUnitBytes, (vi + kMaxPartials2 - 1) / kMaxPartials2});
  return unit_shape(d, d_out, k, es, ti, fine);
}

// Unit shape of the n tokens of one map in the batch-1 kernels: the n tokens
// are n calls of one wave, shaped as a stack plan would shape them (a few
// tokens are latency-bound and take the small units).
static UnitShape linear_shape(const gsi_map *map, int64_t n) {
  const int es = esize_of(map->dtype);
  const int64_t coarse = unit_shape(map->d, map->d_out, map->k, es, 1 << 20).fast_units;
  return shape_in_wave(map->d, map->d_out, map->k, es, (int64_t)map->d * map->k * es * n, coarse * n);
}

static uint64_t linear_ws_bytes(const gsi_map *map, int64_t n) {
  const UnitShape us = linear_shape(map, n);
  return ws_layout(n, n * (us.g_floats + us.part_floats), 0, n * us.a_units).total;
}

// bf16 maps with two or more tokens take the batched MFMA path; fp32 maps
// and single tokens take the batch-1 kernels.
static bool use_batched(const gsi_map *map, int32_t T) { return map->dtype == GSI_BF16 && T >= 2; }

size_t gsi_linear_workspace(const gsi_map *map, int32_t T) {
  if (check_map(map) != GSI_OK || T <= 0) return 0;
  uint64_t need = 0;
  if (use_batched(map, T)) {
    // launches of kMaxBatch tokens, then one with the remainder
    if (T >= kMaxBatch) need = batch_shape(kMaxBatch, map->d, map->k).total;
    if (T % kMaxBatch) {
      const uint64_t r = batch_shape(T % kMaxBatch, map->d, map->k).total;
      if (r > need) need = r;
    }
    return (size_t)need;
  }
  // launches of kMaxCalls tokens, then one with the remainder
  if (T >= kMaxCalls) need = linear_ws_bytes(map, kMaxCalls);
  if (T % kMaxCalls) {
    const uint64_t r = linear_ws_bytes(map, T % kMaxCalls);
    if (r > need) need = r;
  }
  return (size_t)need;
}

static gsi_status linear_batched(const gsi_map *map, const void *x, void *y, int32_t T, float eps,
                                 int32_t mode, float *rho, uint8_t *slow, void *ws,
                                 hipStream_t st) {
  for (int32_t t0 = 0; t0 < T; t0 += kMaxBatch) {
    const int32_t n = (T - t0) < kMaxBatch ? (T - t0) : kMaxBatch;
    const BatchShape b = batch_shape(n, map->d, map->k);
    BArgs a{};
    a.W = map->W;
    a.V = map->V;
    a.M = map->M;
    a.G = map->G;
    a.x = static_cast<const char *>(x) + (int64_t)t0 * map->d * 2;
    a.y = static_cast<char *>(y) + (int64_t)t0 * map->d_out * 2;
    a.rho = rho ? rho + t0 : nullptr;
    a.slow = slow ? slow + t0 : nullptr;
    a.n = n;
    a.d = map->d;
    a.d_out = map->d_out;
    a.k = map->k;
    a.kpad = b.kpad;
    a.kc = b.kc;
    a.splits = b.splits;
    a.mode = mode;
    a.eps = eps;
    char *w = static_cast<char *>(ws);
    a.part = reinterpret_cast<float *>(w + b.part_off);
    a.xxp = reinterpret_cast<float *>(w + b.xxp_off);
    a.ghi = reinterpret_cast<uint16_t *>(w + b.ghi_off);
    a.glo = reinterpret_cast<uint16_t *>(w + b.glo_off);
    a.flags = reinterpret_cast<int32_t *>(w + b.flags_off);
    a.zeros = w + b.zeros_off;
    if (launch_batched(a, st) != hipSuccess) return GSI_E_HIP;
  }
  return GSI_OK;
}

gsi_status gsi_linear(const gsi_map *map, const void *x, void *y, int32_t T, float eps,
                      int32_t mode, float *rho, uint8_t *slow, void *ws, size_t ws_bytes,
                      void *stream) {
  gsi_status s = check_map(map);
  if (s != GSI_OK) return s;
  if (T < 0) return GSI_E_SHAPE;
  if (mode < GSI_GATED || mode > GSI_FORCE_SLOW) return GSI_E_ARG;
  if (T == 0) return GSI_OK;
  if (!x || !y || !ws) return GSI_E_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256) || (rho && !aligned(rho, 4)))
    return GSI_E_ALIGN;
  const size_t need = gsi_linear_workspace(map, T);
  if (ws_bytes < need) return GSI_E_WORKSPACE;

  const int es = esize_of(map->dtype);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_batched(map, T)) return linear_batched(map, x, y, T, eps, mode, rho, slow, ws, st);
  // Tokens are processed in launches of at most kMaxCalls tokens; each
  // launch reuses the same workspace (stream order separates them).
  for (int32_t t0 = 0; t0 < T; t0 += kMaxCalls) {
    const int32_t n = (T - t0) < kMaxCalls ? (T - t0) : kMaxCalls;
    const UnitShape us = linear_shape(map, n);
    const WsLayout wl = ws_layout(n, n * (us.g_floats + us.part_floats), 0, n * us.a_units);
    KArgs a{};
    a.table = nullptr;
    a.unit_call = nullptr;
    CallDesc &o = a.one;
    o.W = map->W;
    o.V = map->V;
    o.M = map->M;
    o.G = map->G;
    o.x = static_cast<const char *>(x) + (int64_t)t0 * map->d * es;
    o.y = static_cast<char *>(y) + (int64_t)t0 * map->d_out * es;
    o.rho = rho ? rho + t0 : nullptr;
    o.slow = slow ? slow + t0 : nullptr;
    o.d = map->d;
    o.d_out = map->d_out;
    o.k = map->k;
    o.eps = eps;
    o.a_begin = 0;
    o.a_units = us.a_units;
    o.a_rows = us.a_rows;
    o.fast_units = us.fast_units;
    o.fast_tiles = us.fast_tiles;
    o.slow_units = us.slow_units;
    o.slow_rows = us.slow_rows;
    o.groups = us.groups;
    o.g_off = 0;
    o.part_off = (int64_t)n * us.g_floats;
    o.gate_off = 0;
    a.x_stride = (int64_t)map->d * es;
    a.y_stride = (int64_t)map->d_out * es;
    a.n = n;
    a.units_a = n * us.a_units;
    a.mode = mode;
    a.max_k = map->k;
    a.max_d = map->d;
    set_ws(a, ws, wl.gate_off, wl.need_off, wl.pref_off, wl.float_off, wl.gcnt_off);
    const int64_t ub = (int64_t)n * (us.fast_units > us.slow_units ? us.fast_units : us.slow_units);
    const hipError_t e = launch_batch1(map->dtype, a, apply_grid(ub), 3, st);
    if (e != hipSuccess) return GSI_E_HIP;
  }
  return GSI_OK;
}

// ---- stacks ----------------------------------------------------------------

static gsi_status check_call(const gsi_call &c, int32_t dtype) {
  gsi_status s = check_map(&c.map);
  if (s != GSI_OK) return s;
  if (c.map.dtype != dtype) return GSI_E_DTYPE;
  if (!c.x || !c.y) return GSI_E_NULL;
  if (!aligned(c.x, 16) || !aligned(c.y, 16) || (c.rho && !aligned(c.rho, 4))) return GSI_E_ALIGN;
  return GSI_OK;
}

// Byte ranges [lo, hi) of one call's x and y.
struct Span {
  uintptr_t lo, hi;
  int32_t call;
};

// Calls of one wave may not write what another call of the same wave reads
// or writes (they run concurrently); across waves anything goes, because a
// wave starts only after the previous one has finished.
static gsi_status check_wave_aliasing(const gsi_call *calls, int32_t b, int32_t e) {
  const int es = esize_of(calls[b].map.dtype);
  std::vector<Span> ys;
  ys.reserve(e - b);
  for (int32_t i = b; i < e; ++i) {
    const uintptr_t y = reinterpret_cast<uintptr_t>(calls[i].y);
    ys.push_back({y, y + (uintptr_t)calls[i].map.d_out * es, i});
  }
  std::sort(ys.begin(), ys.end(), [](const Span &p, const Span &q) { return p.lo < q.lo; });
  for (size_t i = 1; i < ys.size(); ++i)
    if (ys[i].lo < ys[i - 1].hi) return GSI_E_ARG;  // two outputs overlap
  // outputs are now disjoint and sorted by start (and end): for each input,
  // the last output starting below its end is the only candidate overlap
  for (int32_t i = b; i < e; ++i) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(calls[i].x);
    const uintptr_t hi = lo + (uintptr_t)calls[i].map.d * es;
    auto it = std::lower_bound(ys.begin(), ys.end(), hi,
                               [](const Span &p, uintptr_t v) { return p.lo < v; });
    if (it != ys.begin() && std::prev(it)->hi > lo) return GSI_E_ARG;
  }
  return GSI_OK;
}

// For each call, the earlier call of the same wave whose projection it
// shares (same x, V_k, E, d and k: g, ||x|| and rho are then the same), or -1.
static std::vector<int32_t> share_owners(const gsi_call *calls, int32_t n) {
  std::vector<int32_t> owner(n, -1);
  std::map<std::tuple<int32_t, const void *, const void *, const void *, int32_t, int32_t>, int32_t> first;
  for (int32_t i = 0; i < n; ++i) {
    const auto key = std::make_tuple(calls[i].wave, calls[i].x, calls[i].map.V, (const void *)calls[i].map.G,
                                     calls[i].map.d, calls[i].map.k);
    const auto it = first.find(key);
    if (it == first.end())
      first.emplace(key, i);
    else
      owner[i] = it->second;
  }
  return owner;
}

static std::vector<UnitShape> call_shapes(const gsi_call *calls, int32_t n, int es) {
  std::vector<UnitShape> shapes(n);
  const std::vector<int32_t> owner = share_owners(calls, n);
  for (int32_t b = 0; b < n;) {
    int32_t e = b + 1;
    while (e < n && calls[e].wave == calls[b].wave) ++e;
    int64_t vbytes = 0, fast_units = 0;
    for (int32_t i = b; i < e; ++i) {
      if (owner[i] < 0) vbytes += (int64_t)calls[i].map.d * calls[i].map.k * es;
      fast_units += unit_shape(calls[i].map.d, calls[i].map.d_out, calls[i].map.k, es, 1 << 20).fast_units;
    }
    for (int32_t i = b; i < e; ++i) {
      shapes[i] = shape_in_wave(calls[i].map.d, calls[i].map.d_out, calls[i].map.k, es, vbytes, fast_units);
      if (owner[i] >= 0) {  // projected by its owner
        shapes[i].a_units = 0;
        shapes[i].groups = 1;
        shapes[i].part_floats = 0;
      }
    }
    b = e;
  }
  return shapes;
}

static gsi_status plan_sizes(const gsi_call *calls, int32_t n, int64_t *units_a,
                             int64_t *target, size_t *bytes, int32_t *n_waves) {
  if (n < 0 || n > kMaxCalls) return GSI_E_SHAPE;
  if (n > 0 && !calls) return GSI_E_NULL;
  const int32_t dtype = n > 0 ? calls[0].map.dtype : GSI_BF16;
  int64_t vbytes = 0;
  int32_t waves = 0;
  for (int32_t i = 0; i < n; ++i) {
    const gsi_status s = check_call(calls[i], dtype);
    if (s != GSI_OK) return s;
    if (calls[i].wave < 0 || (i > 0 && calls[i].wave < calls[i - 1].wave)) return GSI_E_ARG;
    if (i == 0 || calls[i].wave != calls[i - 1].wave) ++waves;
    vbytes += (int64_t)calls[i].map.d * calls[i].map.k * esize_of(dtype);
  }
  for (int32_t b = 0; b < n;) {
    int32_t e = b + 1;
    while (e < n && calls[e].wave == calls[b].wave) ++e;
    const gsi_status s = check_wave_aliasing(calls, b, e);
    if (s != GSI_OK) return s;
    b = e;
  }
  *n_waves = waves;
  int64_t ua = 0;
  for (const UnitShape &us : call_shapes(calls, n, esize_of(dtype))) ua += us.a_units;
  *units_a = ua;
  *target = plan_proj_target(vbytes);
  const uint64_t desc_off = align_up(sizeof(PlanHeader), 128);
  const uint64_t unit_off = desc_off + (uint64_t)n * sizeof(CallDesc);
  const uint64_t order_off = align_up(unit_off + (uint64_t)ua * 4, 16);
  *bytes = (size_t)align_up(order_off + (uint64_t)(n + 2 * (waves + 1)) * 4, 256);
  return GSI_OK;
}

size_t gsi_stack_plan_bytes(const gsi_call *calls, int32_t n) {
  int64_t ua = 0, t = 0;
  size_t bytes = 0;
  int32_t waves = 0;
  if (plan_sizes(calls, n, &ua, &t, &bytes, &waves) != GSI_OK) return 0;
  return bytes;
}

gsi_status gsi_stack_plan(const gsi_call *calls, int32_t n, void *plan, size_t plan_bytes) {
  int64_t ua = 0, target = 0;
  size_t bytes = 0;
  int32_t n_waves = 0;
  const gsi_status s = plan_sizes(calls, n, &ua, &target, &bytes, &n_waves);
  if (s != GSI_OK) return s;
  if (!plan) return GSI_E_NULL;
  if (!aligned(plan, 16)) return GSI_E_ALIGN;
  if (plan_bytes < bytes) return GSI_E_WORKSPACE;
  std::memset(plan, 0, bytes);
  auto *h = static_cast<PlanHeader *>(plan);
  h->magic = kPlanMagic;
  h->version = kPlanVersion;
  h->n = n;
  h->dtype = n > 0 ? calls[0].map.dtype : GSI_BF16;
  h->desc_off = align_up(sizeof(PlanHeader), 128);
  h->unit_off = h->desc_off + (uint64_t)n * sizeof(CallDesc);
  h->total_bytes = bytes;
  auto *desc = reinterpret_cast<CallDesc *>(static_cast<char *>(plan) + h->desc_off);
  auto *unit_call = reinterpret_cast<int32_t *>(static_cast<char *>(plan) + h->unit_off);
  const int es = esize_of(h->dtype);
  // float offsets: g of every call first, then the partials
  int64_t g_total = 0;
  for (int32_t i = 0; i < n; ++i) g_total += (calls[i].map.k + 3) / 4 * 4;
  // Wave by wave, the projection units of the calls with the most units go
  // first: their final reductions are the longest and should not be the
  // tail.  Outputs are handed out in the same call order, which is the order
  // in which the gates are expected to open.
  std::vector<int32_t> wave_of(n);
  for (int32_t i = 0, w = -1; i < n; ++i) {
    if (i == 0 || calls[i].wave != calls[i - 1].wave) ++w;
    wave_of[i] = w;
  }
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  const std::vector<UnitShape> shapes = call_shapes(calls, n, es);
  const std::vector<int32_t> owner = share_owners(calls, n);
  std::vector<int32_t> nunits(n);
  for (int32_t i = 0; i < n; ++i) nunits[i] = shapes[i].a_units;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    if (wave_of[x] != wave_of[y]) return wave_of[x] < wave_of[y];
    return nunits[x] > nunits[y];
  });
  std::vector<int32_t> first_unit(n);
  {
    int64_t u = 0;
    for (int32_t i : order) {
      first_unit[i] = (int32_t)u;
      u += nunits[i];
    }
  }
  int64_t g_off = 0, part_off = g_total, a_begin = 0, units_b = 0;
  int32_t max_k = 8, max_d = 8, units_max = 1;
  for (int32_t i = 0; i < n; ++i) {
    const gsi_call &c = calls[i];
    const UnitShape &us = shapes[i];
    a_begin = first_unit[i];
    CallDesc &o = desc[i];
    o.W = c.map.W;
    o.V = c.map.V;
    o.M = c.map.M;
    o.G = c.map.G;
    o.x = c.x;
    o.y = c.y;
    o.rho = c.rho;
    o.slow = c.slow;
    o.d = c.map.d;
    o.d_out = c.map.d_out;
    o.k = c.map.k;
    o.eps = c.eps;
    o.a_begin = (int32_t)a_begin;
    o.a_units = us.a_units;
    o.a_rows = us.a_rows;
    o.fast_units = us.fast_units;
    o.fast_tiles = us.fast_tiles;
    o.slow_units = us.slow_units;
    o.slow_rows = us.slow_rows;
    o.groups = us.groups;
    o.g_off = owner[i] < 0 ? g_off : desc[owner[i]].g_off;
    o.part_off = part_off;
    o.gate_off = i;
    o.wave = wave_of[i];
    o.flags = (o.wave > 0 ? kCallXCoherent : 0) | (o.wave + 1 < n_waves ? kCallYCoherent : 0);
    for (int32_t q = 0; q < us.a_units; ++q) unit_call[a_begin + q] = i;
    if (owner[i] >= 0) {  // append to the owner's sharing list
      int32_t last = owner[i];
      while (desc[last].share_next) last = desc[last].share_next - 1;
      desc[last].share_next = i + 1;
    } else {
      g_off += us.g_floats;
    }
    part_off += us.part_floats;
    const int32_t ub = us.fast_units > us.slow_units ? us.fast_units : us.slow_units;
    if (ub >= kMaxUnitsPerCall) return GSI_E_SHAPE;
    units_b += ub;
    if (ub > units_max) units_max = ub;
    if (c.map.k > max_k) max_k = c.map.k;
    if (c.map.d > max_d) max_d = c.map.d;
  }
  {
    int64_t ua = 0;
    for (int32_t i = 0; i < n; ++i) ua += nunits[i];
    h->units_a = (int32_t)ua;
  }
  h->units_b = (int32_t)units_b;
  h->units_max = units_max;
  h->max_k = max_k;
  h->max_d = max_d;
  h->n_waves = n_waves;
  // output order and the per-wave tables of the single-launch kernel
  h->order_off = align_up(h->unit_off + (uint64_t)h->units_a * 4, 16);
  auto *a_order = reinterpret_cast<int32_t *>(static_cast<char *>(plan) + h->order_off);
  int32_t *wave_tab = a_order + n;
  for (int32_t i = 0; i < n; ++i) a_order[i] = order[i];
  for (int32_t w = 0, i = 0; w <= n_waves; ++w) {
    while (i < n && wave_of[order[i]] < w) ++i;
    wave_tab[w] = i < n ? first_unit[order[i]] : h->units_a;  // first projection unit
    wave_tab[n_waves + 1 + w] = i;                               // first output slot
  }
  h->ctl_words = (int32_t)ctl_words(n, n_waves);
  const WsLayout wl = ws_layout(n, part_off, h->ctl_words, h->units_a);
  h->ws_bytes = n > 0 ? wl.total : 0;
  h->ws_gate_off = wl.gate_off;
  h->ws_need_off = wl.need_off;
  h->ws_pref_off = wl.pref_off;
  h->ws_float_off = wl.float_off;
  h->ws_ctl_off = wl.ctl_off;
  return GSI_OK;
}

size_t gsi_stack_workspace(const void *plan_host) {
  if (!plan_host) return 0;
  const auto *h = static_cast<const PlanHeader *>(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return 0;
  return (size_t)h->ws_bytes;
}

size_t gsi_stack_status_offset(const void *plan_host) {
  if (!plan_host) return 0;
  const auto *h = static_cast<const PlanHeader *>(plan_host);
  if (h->magic != kPlanMagic || h->version != kPlanVersion || h->n <= 0) return 0;
  return (size_t)(h->ws_ctl_off + 4 * kCtlStatus);
}

// Bound of every device-side wait of the single-launch kernel, in polls of
// a few hundred ns: far beyond any legitimate wait.  GSI_SPIN_LIMIT
// overrides it (tests force the bound to run out).
static int32_t spin_limit() {
  const char *e = std::getenv("GSI_SPIN_LIMIT");
  if (e && *e) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 0 && v < (1L << 30)) return (int32_t)v;
  }
  return 1 << 22;
}

static gsi_status check_plan_run(const PlanHeader *h, const void *plan_dev, int32_t mode, void *ws,
                                 size_t ws_bytes) {
  if (h->magic != kPlanMagic || h->version != kPlanVersion || h->n < 0 || h->n > kMaxCalls)
    return GSI_E_ARG;
  if (mode < GSI_GATED || mode > GSI_FORCE_SLOW) return GSI_E_ARG;
  if (h->n == 0) return GSI_OK;
  if (!plan_dev || !ws) return GSI_E_NULL;
  if (!aligned(plan_dev, 16) || !aligned(ws, 256)) return GSI_E_ALIGN;
  if (ws_bytes < h->ws_bytes) return GSI_E_WORKSPACE;
  return GSI_OK;
}

gsi_status gsi_stack(const void *plan_host, const void *plan_dev, int32_t mode, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!plan_host) return GSI_E_NULL;
  const auto *h = static_cast<const PlanHeader *>(plan_host);
  const gsi_status s = check_plan_run(h, plan_dev, mode, ws, ws_bytes);
  if (s != GSI_OK || h->n == 0) return s;
  const char *pd = static_cast<const char *>(plan_dev);
  char *w = static_cast<char *>(ws);
  FArgs a{};
  a.table = reinterpret_cast<const CallDesc *>(pd + h->desc_off);
  a.unit_call = reinterpret_cast<const int32_t *>(pd + h->unit_off);
  a.a_order = reinterpret_cast<const int32_t *>(pd + h->order_off);
  a.wave_tab = a.a_order + h->n;
  a.ctl = reinterpret_cast<uint32_t *>(w + h->ws_ctl_off);
  a.entries = reinterpret_cast<uint64_t *>(a.ctl + kCtlWave0 + kCtlWaveWords * h->n_waves);
  a.counters = reinterpret_cast<uint32_t *>(w);
  a.gcounters = reinterpret_cast<uint32_t *>(w + gcnt_offset(h->ws_ctl_off, h->ctl_words));
  a.gate = w + h->ws_gate_off;
  a.wsf = reinterpret_cast<float *>(w + h->ws_float_off);
  a.n = h->n;
  a.n_waves = h->n_waves;
  a.max_k = h->max_k;
  a.max_d = h->max_d;
  a.spin_limit = spin_limit();
  a.units_a = h->units_a;
  const hipError_t e = launch_stack(h->dtype, a, mode, h->units_a + h->units_b,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GSI_OK : GSI_E_HIP;
}

gsi_status gsi_stack_phase(const void *plan_host, const void *plan_dev, int32_t mode,
                           int32_t phase, void *ws, size_t ws_bytes, void *stream) {
  if (!plan_host) return GSI_E_NULL;
  const auto *h = static_cast<const PlanHeader *>(plan_host);
  if (phase < 1 || phase > 3) return GSI_E_ARG;
  const gsi_status s = check_plan_run(h, plan_dev, mode, ws, ws_bytes);
  if (s != GSI_OK || h->n == 0) return s;
  if (h->n_waves > 1) return GSI_E_ARG;  // the two-launch form has no wave barriers
  KArgs a{};
  a.table = reinterpret_cast<const CallDesc *>(static_cast<const char *>(plan_dev) + h->desc_off);
  a.unit_call =
      reinterpret_cast<const int32_t *>(static_cast<const char *>(plan_dev) + h->unit_off);
  a.n = h->n;
  a.units_a = h->units_a;
  a.mode = mode;
  a.max_k = h->max_k;
  a.max_d = h->max_d;
  set_ws(a, ws, h->ws_gate_off, h->ws_need_off, h->ws_pref_off, h->ws_float_off,
         gcnt_offset(h->ws_ctl_off, h->ctl_words));
  const hipError_t e = launch_batch1(h->dtype, a, apply_grid(h->units_b), phase,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GSI_OK : GSI_E_HIP;
}

// ---- basis calibration ----------------------------------------------------

static gsi_status check_calib(const gsi_calib *c) {
  if (!c) return GSI_E_NULL;
  const int es = esize_of(c->dtype);
  if (es == 0) return GSI_E_DTYPE;
  if (c->n <= 0 || c->d <= 0 || c->k <= 0 || c->k > c->d || c->k > c->n || c->k > kMaxK) return GSI_E_SHAPE;
  if (c->iters < 0 || c->iters > 1000) return GSI_E_ARG;
  if (!c->A || !c->V0 || !c->V) return GSI_E_NULL;
  if (!aligned(c->A, 16) || !aligned(c->V0, 16) || !aligned(c->V, 16)) return GSI_E_ALIGN;
  return GSI_OK;
}

size_t gsi_calibrate_workspace(const gsi_calib *c) {
  if (check_calib(c) != GSI_OK) return 0;
  return calib_ws_bytes(c->n, c->d, c->k, c->dtype);
}

size_t gsi_calibrate_status_offset(void) { return 0; }

gsi_status gsi_calibrate(const gsi_calib *c, void *ws, size_t ws_bytes, void *stream) {
  const gsi_status s = check_calib(c);
  if (s != GSI_OK) return s;
  if (!ws) return GSI_E_NULL;
  if (!aligned(ws, 256)) return GSI_E_ALIGN;
  if (ws_bytes < calib_ws_bytes(c->n, c->d, c->k, c->dtype)) return GSI_E_WORKSPACE;
  CalibArgs a{};
  a.n = c->n;
  a.d = c->d;
  a.k = c->k;
  a.dtype = c->dtype;
  a.iters = c->iters;
  a.A = c->A;
  a.V0 = c->V0;
  a.V = c->V;
  char *w = static_cast<char *>(ws);
  const CalibLayout L = calib_layout(c->n, c->d, c->k, c->dtype);
  a.status = reinterpret_cast<uint32_t *>(w + L.status);
  a.mfma = L.mfma ? 1 : 0;
  a.dp = (int32_t)L.dp;
  a.np = (int32_t)L.np;
  if (L.mfma) {
    a.zeros = w + L.zeros;
    a.vt3 = reinterpret_cast<uint16_t *>(w + L.vt3);
    a.zt3 = reinterpret_cast<uint16_t *>(w + L.zt3);
    a.at = reinterpret_cast<uint16_t *>(w + L.at);
  } else {
    a.vw = reinterpret_cast<float *>(w + L.vw);
    a.z = reinterpret_cast<float *>(w + L.z);
  }
  a.y = reinterpret_cast<double *>(w + L.y);
  a.y2 = reinterpret_cast<double *>(w + L.y2);
  a.g = reinterpret_cast<double *>(w + L.g);
  a.r = reinterpret_cast<double *>(w + L.r);
  a.dinv = reinterpret_cast<double *>(w + L.dinv);
  a.gpart = reinterpret_cast<double *>(w + L.gpart);
  const hipError_t e = launch_calibrate(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GSI_OK : GSI_E_HIP;
}

}  // extern "C"
