/*
 * gsi.h -- C ABI of libgsi, the gated subspace linear map on MI355X (gfx950).
 *
 * Method: "Gated Subspace Inference for Transformer Acceleration"
 * (S. J. Thomas, 2026), technical summary (cited as GSI-TS):
 *   - §2.1 core decomposition: x = V_k V_k^T x + r, y = W x = M g + W r with
 *     the cached image M = W V_k (d_out x k) and g = V_k^T x (k values);
 *   - §2.2 gated residual step: per token rho = ||r|| / ||x||; if rho < eps
 *     the output is y = M g (fast path), otherwise y = W x (slow path);
 *   - §3 the gate is applied to every linear map of a transformer.
 *
 * Conventions shared by every entry point
 *   - Every buffer is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t, NULL for
 *     the default stream); results are valid once the caller synchronises
 *     that stream.  No entry point synchronises the host.
 *   - Arguments are checked on the host before any launch; a non-OK status
 *     means nothing was enqueued (except GSI_E_HIP, reported after a launch
 *     failed).  Nothing is printed, nothing aborts.
 *   - Storage dtype: GSI_FP32 or GSI_BF16 for W, V_k, M, x and y alike.
 *     Accumulation is fp32 everywhere; g, norms and rho are fp32.
 *   - Shapes: d, d_out, k positive multiples of 8, k <= min(d, 1024),
 *     d * sizeof(element) <= 32 KiB (x is staged in LDS).
 *   - Alignment: W, V_k, M, G, x, y 16-byte aligned; rho 4-byte aligned.
 *   - Gate (GSI-TS §2.2): slow = !(rho < eps).  Ties go slow; ||x|| = 0
 *     gives rho = 0; a NaN/Inf token gives rho = NaN and goes slow.
 *     On the GPU rho is evaluated as sqrt(max(0, 1 - ||g||^2/||x||^2)),
 *     which equals ||x - V_k g|| / ||x|| for an orthonormal V_k, or exactly
 *     for the stored basis when the map carries E (gsi_map.G).
 */
#ifndef GSI_H
#define GSI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSI_ABI_VERSION 3

typedef enum {
  GSI_OK = 0,
  GSI_E_NULL = 1,      /* a required pointer is NULL                          */
  GSI_E_SHAPE = 2,     /* d, d_out, k, T or n outside the documented limits   */
  GSI_E_DTYPE = 3,     /* unknown dtype, or mixed dtypes in one stack         */
  GSI_E_ALIGN = 4,     /* a pointer is not aligned as documented              */
  GSI_E_WORKSPACE = 5, /* workspace smaller than the matching *_workspace()   */
  GSI_E_HIP = 6,       /* the HIP runtime reported an error                   */
  GSI_E_ARG = 7,       /* bad mode, bad plan or other invalid argument        */
} gsi_status;

typedef enum { GSI_FP32 = 0, GSI_BF16 = 1 } gsi_dtype;

typedef enum {
  GSI_GATED = 0,       /* per-token gate of GSI-TS §2.2                        */
  GSI_FORCE_FAST = 1,  /* always y = M g: the static projection control (§4) */
  GSI_FORCE_SLOW = 2,  /* always y = W x: the dense baseline                   */
} gsi_mode;

/* One linear map y = W x with its basis and cached image.
 *   W : [d_out][d] row-major (the nn.Linear layout)
 *   V : [d][k] row-major, orthonormal columns (the basis V_k)
 *   M : the image M = W V_k in the library's tiled layout, gsi_image_bytes()
 *       bytes, written by gsi_prepare.  Tiled layout: element (i, j) of the
 *       d_out x k image lives at
 *         ((i / 64) * (k / VW) + j / VW) * 64 * VW + (i % 64) * VW + j % VW
 *       with VW = 16 / sizeof(element) (8 for bf16, 4 for fp32); the rows
 *       of the last 64-row tile beyond d_out hold zeros.  A wavefront of 64
 *       lanes thus reads one 16-byte vector of 64 consecutive rows at once. */
typedef struct gsi_map {
  int32_t d;
  int32_t d_out;
  int32_t k;
  int32_t dtype;   /* gsi_dtype */
  const void *W;
  const void *V;
  void *M;
  /* Optional (NULL for none): E = V_k^T V_k - I, [k][k] row-major in the
   * storage dtype, gsi_gram_bytes() bytes, written by gsi_prepare.  With it
   * every gate of the map uses the residual ratio exactly for the stored
   * basis, rho = sqrt(max(0, ||x||^2 - ||g||^2 + g^T E g)) / ||x||, which is
   * ||x - V_k g|| / ||x|| (GSI-TS §2.2) even where rounding has left V_k only
   * nearly orthonormal; without it rho = sqrt(1 - ||g||^2/||x||^2), exact
   * only for an orthonormal V_k.  Costs one read of E per gate. */
  void *G;
} gsi_map;

/* One batch-1 call of a stack: one token x [d] -> y [d_out] through `map`.
 * rho (one float) and slow (one byte, 1 = slow path taken) may be NULL.
 * wave: calls of a stack run in waves (see gsi_stack); 0 for a stack of
 * independent calls. */
typedef struct gsi_call {
  gsi_map map;
  const void *x;
  void *y;
  float eps;
  int32_t wave;
  float *rho;
  uint8_t *slow;
} gsi_call;

/* ABI version compiled into the library (GSI_ABI_VERSION). */
int32_t gsi_abi_version(void);

/* Static, NUL-terminated name of a status code. */
const char *gsi_status_str(int32_t status);

/* Bytes of the cached image M of a d_out x k map in the tiled layout above,
 * or 0 for invalid arguments. */
size_t gsi_image_bytes(int32_t d_out, int32_t k, int32_t dtype);

/* Bytes of E = V_k^T V_k - I of a map with k basis columns (see gsi_map.G),
 * or 0 for invalid arguments. */
size_t gsi_gram_bytes(int32_t k, int32_t dtype);

/* Build the cached image M = W V_k (GSI-TS §2.1) into map->M, and, if
 * map->G is set, E = V_k^T V_k - I into map->G.  fp32 accumulation, rounded
 * to nearest-even into the storage dtype; the padding rows of the last tile
 * of M are written as zeros.  Runs once per map, off the per-token path. */
gsi_status gsi_prepare(const gsi_map *map, void *stream);

/* Workspace bytes gsi_linear needs for T tokens of `map` (0 if T == 0). */
size_t gsi_linear_workspace(const gsi_map *map, int32_t T);

/* Gated map on T tokens (GSI-TS §2.1-§2.2).
 *   x   : [T][d] device, y : [T][d_out] device (written for every token)
 *   eps : threshold; mode : gsi_mode
 *   rho : [T] floats or NULL; slow : [T] bytes or NULL
 *   ws  : device workspace of at least gsi_linear_workspace(map, T) bytes.
 *         It must be zero-filled before its first use; every call leaves
 *         its counters at zero again, so the same buffer can be reused by
 *         later calls on the same stream.  Calls that share a workspace
 *         must not run concurrently.
 * T == 0 is a no-op returning GSI_OK.  Tokens are independent: the result
 * of a token does not depend on the other tokens of the batch. */
gsi_status gsi_linear(const gsi_map *map, const void *x, void *y, int32_t T, float eps,
                      int32_t mode, float *rho, uint8_t *slow, void *ws, size_t ws_bytes,
                      void *stream);

/* ---- gsi_linear without caller memory ----
 * For callers that cannot allocate: code under HIP graph capture, serving
 * loops that may not call hipMalloc, harnesses that forbid allocation.
 * gsi_linear_static is gsi_linear (same kernels, same results) with its
 * workspace in a device array of the library, GSI_STATIC_SCRATCH_BYTES
 * (64 MiB) per device, held from library load until the process ends.  It
 * allocates nothing and calls no allocating routine.
 *   - A call whose gsi_linear_workspace(map, T) exceeds the array returns
 *     GSI_E_WORKSPACE and enqueues nothing (e.g. T = 256 fits up to
 *     d = 16384, k = 512; larger batches can be split by the caller).
 *   - Each call first clears the part of the array it uses with a fill
 *     kernel on `stream` (no memset node), then enqueues gsi_linear's
 *     kernels; all arguments but the workspace are as for gsi_linear.
 *   - Every call on one device shares that device's array: calls that may
 *     overlap on one device (different streams without ordering) race and
 *     must not be issued. */
#define GSI_STATIC_SCRATCH_BYTES (64u << 20)

/* Bytes of the library's device array (GSI_STATIC_SCRATCH_BYTES). */
size_t gsi_static_scratch_bytes(void);

gsi_status gsi_linear_static(const gsi_map *map, const void *x, void *y, int32_t T, float eps,
                             int32_t mode, float *rho, uint8_t *slow, void *stream);

/* ---- stacks: every linear map of a decode step in one launch (GSI-TS §3) ----
 * A stack plan is built once on the host from an array of calls and copied
 * by the caller to device memory; running the plan is one kernel launch.
 * Calls of one stack share one dtype.
 *
 * Waves: calls carry a wave number, nondecreasing along the array.  The
 * calls of one wave run concurrently and must be independent: no call of a
 * wave may write bytes that another call of the same wave reads (x) or
 * writes (y) -- gsi_stack_plan rejects such overlaps with GSI_E_ARG.  A
 * wave starts only after every call of the previous wave has written its y,
 * so a call may read as its x the y of any call of an earlier wave (a
 * dependency-chained stack such as the layers of a decoder: the QKV and
 * fc_in maps of a GPT-J block in one wave, out and fc_out in the next).
 * The barriers between waves are kept on the device (no host round trip).
 * With every wave number equal, all calls are independent.
 *
 * Why a plan, and why batch 1: a decode step runs the same maps on the same
 * buffers every token, so the call array is validated and laid out once
 * (gsi_stack_plan) and each step is then a single launch with no host-side
 * work (gsi_stack).  A call is one token: at batch 1 every map's bytes are
 * only microseconds of HBM time, so the maps of a step have to overlap in
 * one persistent launch.  For T >= 2 tokens per map, gsi_linear's batched
 * path reads each map once for all its tokens; T tokens through n maps with
 * batch-1 semantics are n * T calls of one plan. */

/* Bytes of the host plan for these n calls (0 if n < 0 or n > 4096, or if
 * a call is invalid; gsi_stack_plan reports which check failed). */
size_t gsi_stack_plan_bytes(const gsi_call *calls, int32_t n);

/* Validate `calls` (host array of n calls holding device pointers) and
 * write the plan into the HOST buffer `plan` of plan_bytes bytes.
 * The plan embeds the device pointers of the calls; a plan stays valid for
 * as long as those buffers do. */
gsi_status gsi_stack_plan(const gsi_call *calls, int32_t n, void *plan, size_t plan_bytes);

/* Workspace bytes needed to run a plan (read from the host plan). */
size_t gsi_stack_workspace(const void *plan_host);

/* Run every call of a plan: plan_host is the host buffer gsi_stack_plan
 * filled, plan_dev a byte-identical device copy of it.  Same workspace
 * rules as gsi_linear.  Equivalent to gsi_linear(T = 1) on each call, in
 * array order; the results are bitwise identical to the two-phase form
 * below for the same plan.  One persistent launch: the output work of a
 * call starts as soon as its own gate is decided, while other calls are
 * still projecting.
 * The launch sizes its grid to what fits on the device at once and relies
 * on all of it being resident (the first tickets of a wave are static, and
 * a wave starts once every workgroup has left the previous one).
 * Every device-side wait of the launch is bounded; if a bound ever ran out
 * (a library fault, or a device whose compute units other kernels hold)
 * the launch still ends, the outputs of that run are incomplete and a
 * nonzero code is left in the 32-bit status word at byte
 * gsi_stack_status_offset(plan_host) of the workspace.  The word stays set
 * until the caller clears it; other runs leave it alone. */
gsi_status gsi_stack(const void *plan_host, const void *plan_dev, int32_t mode, void *ws,
                     size_t ws_bytes, void *stream);

/* Byte offset in the workspace of the status word described above (0 if
 * the plan is invalid or empty). */
size_t gsi_stack_status_offset(const void *plan_host);

/* The two phases of a stack as two launches, for callers that interleave
 * other work between them or time them separately.  Only for plans of one
 * wave (GSI_E_ARG otherwise).
 *   GSI_PHASE_PROJECT : g = V_k^T x, ||x||, rho and the gate of every call
 *                       (GSI-TS §2.1-§2.2); writes rho/slow of each call;
 *   GSI_PHASE_APPLY   : every call's output through the path its gate chose
 *                       (y = M g or y = W x).  Needs the project phase of the
 *                       same plan to have run before it on the same workspace
 *                       and stream order.
 * gsi_stack(...) is gsi_stack_phase(PROJECT) followed by (APPLY). */
typedef enum { GSI_PHASE_PROJECT = 1, GSI_PHASE_APPLY = 2 } gsi_phase;

gsi_status gsi_stack_phase(const void *plan_host, const void *plan_dev, int32_t mode,
                           int32_t phase, void *ws, size_t ws_bytes, void *stream);

/* ---- basis calibration (GSI-TS §2.3) ----
 * The summary computes each layer's basis once from activations of a
 * calibration pass, as the top-k subspace of those activations, and starts
 * layer l+1 from layer l's basis so that only small corrections are needed
 * (the depth cascade).  gsi_calibrate runs `iters` sweeps of block subspace
 * iteration V <- orth(A^T (A V)) from V0: with a random V0 (a cold start)
 * the sweeps converge to the dominant k-dimensional subspace of the samples
 * at the rate of the spectral gap; with the previous layer's basis as V0
 * (the cascade) a few sweeps suffice.  orth() is the Q factor of the block
 * (Q^T Y upper triangular with a positive diagonal, the basis Gram-Schmidt
 * gives), formed by two CholeskyQR passes in fp64; the products with A
 * accumulate in fp32. */
typedef struct gsi_calib {
  int32_t n;        /* activation samples (tokens); k <= n                     */
  int32_t d;        /* their dimension                                         */
  int32_t k;        /* basis columns, k <= min(d, 1024)                        */
  int32_t dtype;    /* gsi_dtype of A, V0 and V                                */
  const void *A;    /* [n][d] row-major samples (device)                       */
  const void *V0;   /* [d][k] starting basis (device); need not be orthonormal */
  void *V;          /* [d][k] output: orthonormal basis (device); may equal V0 */
  int32_t iters;    /* sweeps, 0..1000 (0 copies V0)                           */
  int32_t reserved;
} gsi_calib;

/* Workspace bytes of gsi_calibrate (0 for invalid arguments). */
size_t gsi_calibrate_workspace(const gsi_calib *c);

/* Byte offset in the calibration workspace of its 32-bit status word: 0
 * after a good run, nonzero if a block was numerically rank deficient (V is
 * then not reliable).  The word is not cleared by the library. */
size_t gsi_calibrate_status_offset(void);

/* Run the sweeps (asynchronous on `stream`).  The workspace needs no
 * initial contents except a zero status word. */
gsi_status gsi_calibrate(const gsi_calib *c, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GSI_H */
