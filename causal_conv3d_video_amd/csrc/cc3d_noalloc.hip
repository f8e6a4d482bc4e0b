// causal_conv3d_forward_packed_noalloc: the packed-image forward with its
// split workspace in a static device array instead of caller memory, for
// callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "cc3d_device.h"

namespace {

// The workspace of the no-allocation entry point: one array per device the
// library runs on, held until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[CC3D_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device `dev` (looked up
// with that device current, the first time), or null on failure.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Zeroes n ints (the arrival counters a split call expects at launch).
__global__ __launch_bounds__(256) void clear_ints(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

extern "C" cc3d_status_t causal_conv3d_forward_packed_noalloc(cc3d_plan_t plan, const void* x, const void* cache_in,
                                                              const void* w_packed, const void* b, void* out,
                                                              void* cache_out, void* stream) {
  if (!plan || !w_packed || plan->d.dtype != CC3D_BF16) {
    cc3d::g_invalid.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_INVALID_ARG;
  }
  const int64_t need = plan->info.workspace_bytes;
  if (need > int64_t(CC3D_NOALLOC_SCRATCH_BYTES)) {
    cc3d::g_unsupported.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_UNSUPPORTED;
  }
  if (need == 0)
    return causal_conv3d_forward_packed(plan, x, cache_in, w_packed, b, out, cache_out, nullptr, 0, stream);
  int dev = 0;
  void* ws = nullptr;
  if (hipGetDevice(&dev) != hipSuccess || !(ws = scratch_ptr(dev))) {
    cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_DEVICE;
  }
  // the arrival counters (an int per tile at the start) must be zero: the
  // previous call left them so, but they are cleared anyway, on the stream
  int n = int(plan->info.tiles);
  int* cnt = static_cast<int*>(ws);
  void* args[] = {&cnt, &n};
  if (hipLaunchKernel(reinterpret_cast<const void*>(&clear_ints), dim3((n + 255) / 256), dim3(256), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess) {
    cc3d::g_device_error.fetch_add(1, std::memory_order_relaxed);
    return CC3D_ERR_DEVICE;
  }
  return causal_conv3d_forward_packed(plan, x, cache_in, w_packed, b, out, cache_out, ws,
                                      int64_t(CC3D_NOALLOC_SCRATCH_BYTES), stream);
}
