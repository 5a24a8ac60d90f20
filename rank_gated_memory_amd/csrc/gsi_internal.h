// Internal layout shared by the host library (gsi_api.cpp) and the kernels
// (gsi_kernels.hip).  Nothing here is part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gsi {

constexpr uint32_t kPlanMagic = 0x50495347u;  // "GSIP"
constexpr uint32_t kPlanVersion = 3;
constexpr int kBlock = 256;          // threads per workgroup of every kernel
constexpr int kWaves = kBlock / 64;  // wavefronts per workgroup
constexpr int kTileRows = 64;        // image rows per tile (one per lane)
constexpr int kMaxK = 1024;
constexpr int kMaxRowBytes = 32768;  // d * sizeof(element) limit (x staged in LDS)
constexpr int kMaxCalls = 4096;      // calls per stack / tokens per launch
constexpr int kProjRowsMax = 2048;   // rows of V_k per projection unit (x chunk in LDS)

// Device descriptor of one batch-1 call (one token through one map).
struct alignas(16) CallDesc {
  const void *W;
  const void *V;
  const void *M;
  const void *x;
  void *y;
  float *rho;
  uint8_t *slow;
  int32_t d, d_out, k;
  float eps;
  int32_t a_begin;     // first projection unit of this call
  int32_t a_units;     // projection units (row chunks of V_k)
  int32_t a_rows;      // rows of V_k per projection unit
  int32_t fast_units;  // output units when the fast path is taken
  int32_t slow_units;  // output units when the slow path is taken
  int32_t slow_rows;   // rows of W per slow output unit
  int64_t part_off;    // float offset in the workspace of the partials [a_units][k + 4]
  int64_t g_off;       // float offset in the workspace of g [k]
  int32_t gate_off;    // index of this call's gate record / counter
  int32_t fast_tiles;  // 64-row image tiles per fast output unit (multiple of kWaves, or 1:
                       // one tile whose columns are split over the wavefronts)
  int32_t flags;       // kCallXCoherent | kCallYCoherent
  int32_t wave;        // wave of the call in a stack (0 for independent calls)
  // Calls of one wave with the same x, V_k, d and k share one projection:
  // the first of them (the owner) has the projection units; the others have
  // none, read the owner's g, and have their gates decided by the owner's
  // last projection unit.  share_next = 1 + the next call of the group
  // (0: none), so a zero-filled descriptor shares nothing.
  int32_t share_next;
  int32_t groups;      // partial groups (1: the last unit sums all partials; see kGroupUnits)
  const void *G;       // E = V_k^T V_k - I [k][k] (exact rho), or null (norm form)
};
static_assert(sizeof(CallDesc) == 144, "CallDesc layout");

// CallDesc::flags.  In a stack of several waves, x of a later wave may be
// the y of an earlier one, written inside the same launch by a workgroup on
// another XCD: such x is read, and such y written, with agent-coherent
// accesses (the eight XCD L2s are not coherent with each other).
constexpr int32_t kCallXCoherent = 1;
constexpr int32_t kCallYCoherent = 2;

// Header of a stack plan (host buffer, copied verbatim to the device).
struct alignas(16) PlanHeader {
  uint32_t magic;
  uint32_t version;
  int32_t n;           // calls
  int32_t dtype;       // gsi_dtype of every call
  int32_t units_a;     // projection units over all calls
  int32_t units_b;     // sum over calls of max(fast_units, slow_units)
  int32_t max_k;
  int32_t max_d;
  uint64_t ws_bytes;   // workspace bytes
  uint64_t desc_off;   // byte offset of CallDesc[n]
  uint64_t unit_off;   // byte offset of int32 unit_call[units_a]
  uint64_t total_bytes;
  uint64_t ws_gate_off;  // byte offsets of the workspace regions
  uint64_t ws_need_off;
  uint64_t ws_pref_off;
  uint64_t ws_float_off;
  uint64_t ws_ctl_off;   // control words of the single-launch stack kernel
  uint64_t order_off;    // int32 a_order[n], then int32 wave_tab[2 (n_waves + 1)]
  int32_t n_waves;
  int32_t ctl_words;
  int32_t units_max;     // largest per-call max(fast_units, slow_units)
  int32_t pad_;
};
static_assert(sizeof(PlanHeader) == 128, "PlanHeader layout");

// Control words of the single-launch stack kernel (uint32, zero between
// launches except the status word).  Hot words sit on separate 128-byte
// lines.
constexpr int kCtlStatus = 0;       // sticky: nonzero once a device-side wait ran out
constexpr int kCtlExit = 32;        // workgroups that have left the work loop
constexpr int kCtlSeg = 64;         // first work segment not known to be exhausted
constexpr int kCtlWave0 = 96;       // per wave: kCtlWaveWords words, then the open lists
// Ticket and completion counters are split into kGroups copies, one per
// group of workgroups (blockIdx % kGroups), each on its own line: one
// address taking every workgroup's atomics serialises them (~13 ns each).
constexpr int kGroups = 8;
constexpr int kCtlWaveWords = (4 * kGroups + 2) * 32;
constexpr int kWvProj = 0;               // + 32 g: projection tickets taken by group g
constexpr int kWvOut = 32 * kGroups;     // + 32 g: output tickets taken by group g
constexpr int kWvLeft = 64 * kGroups;    // + 32 g: workgroups of group g that have left the wave
constexpr int kWvReady = 96 * kGroups;   // + 32 g: 1 once every workgroup has left (a copy per group)
constexpr int kWvOpen = 128 * kGroups;   // open word (64-bit): calls open << 40 | their output units
constexpr int kWvGroups = 128 * kGroups + 32;  // groups whose workgroups have all left
// After the wave blocks: the open list, one 64-bit entry per call, indexed by
// the wave's first a_order slot plus the order in which the call's gate
// opened: base | need << 32 | slow << 50 | (call + 1) << 51, where base is
// the wave's output ticket of the call's first unit and need its unit count.
constexpr int kEntryNeedBits = 18;
constexpr int64_t kMaxUnitsPerCall = (int64_t)1 << kEntryNeedBits;
inline int64_t ctl_words(int64_t n, int64_t n_waves) {
  return kCtlWave0 + kCtlWaveWords * n_waves + 2 * n;
}

// Workspace regions (byte offsets from the workspace base):
//   [0, 4(n+1))         uint32 counters: one per call, then one for the whole
//                       launch (all zero between launches)
//   [gate_off, +16n)    float4 gate record per call: rho, slow flag bits, ||x||^2, ||g||^2
//   [need_off, +4n)     int32 output units the chosen path of each call needs
//   [pref_off, +4(n+1)) int32 exclusive prefix of need (pref[n] = all units)
//   [float_off, ...)    floats: g of every call, then projection partials
#if defined(__HIPCC__)
__host__ __device__
#endif
inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Arguments of the two batch-1 kernels.  Either `table` points at the
// device copy of a plan's CallDesc array (stack), or it is null and the n
// calls are the n tokens of one map described by `one` (single map, token
// stride x_stride / y_stride elements).
struct KArgs {
  const CallDesc *table;
  const int32_t *unit_call;
  CallDesc one;
  int64_t x_stride;
  int64_t y_stride;
  int32_t n;
  int32_t units_a;
  int32_t mode;
  int32_t max_k;
  int32_t max_d;
  int32_t pad_;
  uint32_t *counters;
  uint32_t *gcounters;  // group counters of two-level partial sums (index a_begin + group)
  void *gate;   // float4 records
  int32_t *need;
  int32_t *pref;
  float *wsf;
};

// Arguments of the single-launch stack kernel.  Work is a sequence of
// segments: the projection units of wave 0, the output units of wave 0, the
// projection units of wave 1, ...  Workgroups take tickets segment by
// segment; see stack_kernel.
struct FArgs {
  const CallDesc *table;
  const int32_t *unit_call;  // projection unit -> call, wave-major
  const int32_t *a_order;    // calls in output order, wave-major
  const int32_t *wave_tab;   // [n_waves + 1] first projection unit of each wave,
                             // then [n_waves + 1] first a_order slot of each wave
  uint32_t *ctl;             // control words (kCtl*)
  uint64_t *entries;         // open lists: ctl + kCtlWave0 + kCtlWaveWords * n_waves
  uint32_t *counters;        // per-call projection counters
  uint32_t *gcounters;       // group counters of two-level partial sums (index a_begin + group)
  void *gate;                // float4 records
  float *wsf;
  int32_t n;
  int32_t n_waves;
  int32_t max_k;
  int32_t max_d;
  int32_t spin_limit;        // bound of every device-side wait (polls)
  int32_t units_a;           // projection units of the plan (entries of gcounters)
};

// A call with more than kGroupUnits2 projection units sums its partials in
// two levels: the last unit of each group of kGroupUnits sums the group into
// a group partial (stored after the unit partials), and the last group to
// finish sums the group partials.  One workgroup then never sums more than
// 64 rows, so a wide V_k can be split into many small units.
constexpr int kGroupUnits = 16;
constexpr int kGroupUnits2 = 64;

// Unit sizing shared by the stack plan and the single-map path.
struct UnitShape {
  int32_t a_units, a_rows, fast_units, fast_tiles, slow_units, slow_rows, groups;
  int64_t part_floats;  // (a_units + group partials) * (k + 4)
  int64_t g_floats;     // k rounded up to a multiple of 4
};

// Output units aim at this many bytes of M (fast) or W (slow), so that a
// contiguous range of units is a balanced share of a launch.
#ifndef GSI_APPLY_UNIT_KB
#define GSI_APPLY_UNIT_KB 256
#endif
constexpr int64_t kApplyUnitBytes = GSI_APPLY_UNIT_KB * 1024;
// Slow units stage x (up to 32 KiB) once per unit: larger units amortise it.
#ifndef GSI_SLOW_UNIT_KB
#define GSI_SLOW_UNIT_KB 256
#endif
constexpr int64_t kSlowUnitBytes = GSI_SLOW_UNIT_KB * 1024;

// fine: latency-bound waves (few bytes per wave) take the smallest fast
// output units, one 64-row image tile whose columns are split over the
// wavefronts of a workgroup, so that every workgroup of the launch gets a
// share of a small wave.  Slow units keep their size: a slow call reads all
// of W and is bandwidth-bound even alone.
inline UnitShape unit_shape(int d, int d_out, int k, int esize, int64_t target_proj_bytes,
                            bool fine = false) {
  UnitShape s{};
  const int64_t row_bytes = (int64_t)k * esize;
  int64_t rows = target_proj_bytes / row_bytes;
  rows = (rows + 15) / 16 * 16;
  if (rows < 16) rows = 16;
  if (rows > kProjRowsMax) rows = kProjRowsMax;
  if (rows > d) rows = d;
  s.a_rows = (int32_t)rows;
  s.a_units = (int32_t)((d + rows - 1) / rows);
  const int tiles = (d_out + kTileRows - 1) / kTileRows;
  int64_t ft = kApplyUnitBytes / ((int64_t)kTileRows * k * esize);
  ft = (ft + kWaves - 1) / kWaves * kWaves;
  if (ft < kWaves) ft = kWaves;
  if (ft > 8 * kWaves) ft = 8 * kWaves;
  if (fine) ft = 1;
  s.fast_tiles = (int32_t)ft;
  s.fast_units = (int32_t)((tiles + ft - 1) / ft);
  int64_t srows = kSlowUnitBytes / ((int64_t)d * esize);
  srows = srows / kWaves * kWaves;
  if (srows < kWaves) srows = kWaves;
  if (srows > 256) srows = 256;
  s.slow_rows = (int32_t)srows;
  s.slow_units = (int32_t)((d_out + srows - 1) / srows);
  s.groups = s.a_units > kGroupUnits2 ? (s.a_units + kGroupUnits - 1) / kGroupUnits : 1;
  s.part_floats = (int64_t)(s.a_units + (s.groups > 1 ? s.groups : 0)) * (k + 4);
  s.g_floats = (k + 3) / 4 * 4;
  return s;
}

}  // namespace gsi
