// gsi_linear_static: the gated map of gsi_linear with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under HIP graph capture, serving loops that forbid
// hipMalloc).  Same kernels and results as gsi_linear.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gsi.h"

namespace {

// One copy per device, held from module load until the process ends.
constexpr size_t kScratchBytes = (size_t)GSI_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Zero n bytes (n a multiple of 16) at p: 16-byte vector stores, grid-stride.
__global__ void __launch_bounds__(256) zero_kernel(uint4 *p, size_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (the array's host-side name is not a
// device address and must never reach a kernel).
gsi_status scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GSI_E_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GSI_E_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GSI_OK;
}

}  // namespace

extern "C" {

size_t gsi_static_scratch_bytes(void) { return kScratchBytes; }

gsi_status gsi_linear_static(const gsi_map *map, const void *x, void *y, int32_t T, float eps,
                             int32_t mode, float *rho, uint8_t *slow, void *stream) {
  if (!map) return GSI_E_NULL;
  if (T < 0) return GSI_E_SHAPE;
  if (T == 0) return gsi_linear(map, x, y, 0, eps, mode, rho, slow, nullptr, 0, stream);
  const size_t need = gsi_linear_workspace(map, T);
  if (need == 0) {
    // invalid map or arguments: let gsi_linear name the failing check
    return gsi_linear(map, x, y, T, eps, mode, rho, slow, nullptr, 0, stream);
  }
  if (need > kScratchBytes) return GSI_E_WORKSPACE;
  // gsi_linear's own argument checks, before anything is enqueued (the
  // clear below must not run for a call that is then rejected)
  if (mode < GSI_GATED || mode > GSI_FORCE_SLOW) return GSI_E_ARG;
  if (!x || !y) return GSI_E_NULL;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 16 ||
      (rho && reinterpret_cast<uintptr_t>(rho) % 4))
    return GSI_E_ALIGN;
  void *ws = nullptr;
  const gsi_status s = scratch_ptr(&ws);
  if (s != GSI_OK) return s;
  // gsi_linear wants a zero-filled workspace; clear the part this call uses
  // with a fill kernel on the caller's stream (no memset node, no host sync).
  const size_t n16 = (need + 15) / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4 *>(ws), n16);
  if (hipGetLastError() != hipSuccess) return GSI_E_HIP;
  return gsi_linear(map, x, y, T, eps, mode, rho, slow, ws, kScratchBytes, stream);
}

}  // extern "C"
