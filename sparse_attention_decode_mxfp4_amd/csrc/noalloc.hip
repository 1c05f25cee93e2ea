// decode_step_noalloc: decode_step with its workspace in a device array that
// the library itself holds, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). The array, `scratch`, is a file-scope device variable: each
// GPU the library runs on holds one copy of MXS_NOALLOC_SCRATCH_BYTES bytes
// until the process ends. Its device address is taken once per device with
// hipGetSymbolAddress (the host-side name of the array is not a device
// address) and kept; the call then runs decode_step's validation and launch
// chain over that address. Nothing is allocated or freed.
//
// decode_step's workspace needs no initialization (its first launch clears
// the merge counters, each row's merging workgroup sets its counter back to
// zero), so the array's contents left by an earlier call do not matter. All
// calls on one GPU share its array: calls that overlap on one GPU (two
// streams, two threads) race on it and must be serialized by the caller.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "launch.hpp"
#include "mxsparse.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MXS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The device address of `scratch` on `dev` (the current device), looked up
// on the first call for that device.
hipError_t scratch_ptr(int dev, void **ptr) {
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_status[dev];
}

}  // namespace

extern "C" int decode_step_noalloc(const mxs_step *step, void *stream) {
  char msg[256];
  if (!step) return mxs::api_error(MXS_EINVAL, "step: null");
  const int32_t P = step->num_partitions != 0
                        ? step->num_partitions
                        : mxs_default_partitions_for(step->B, step->q, step->topk, step->cache.kv_format);
  const size_t need = mxs_workspace_bytes(step->B, step->q, step->H, step->H_I, step->topk,
                                          step->cache.page_table_stride, P);
  if (need > (size_t)MXS_NOALLOC_SCRATCH_BYTES) {
    snprintf(msg, sizeof msg,
             "decode_step_noalloc: the step needs %zu bytes of workspace, more than the library's "
             "scratch of %zu bytes (use decode_step with a caller workspace)",
             need, (size_t)MXS_NOALLOC_SCRATCH_BYTES);
    return mxs::api_error(MXS_EWORKSPACE, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof msg, "decode_step_noalloc: no usable current device (%d: %s)", dev, hipGetErrorString(e));
    return mxs::api_error(MXS_ELAUNCH, msg);
  }
  void *ws = nullptr;
  e = scratch_ptr(dev, &ws);
  if (e != hipSuccess || !ws) {
    snprintf(msg, sizeof msg, "decode_step_noalloc: device address of the scratch array on device %d: %s", dev,
             hipGetErrorString(e));
    return mxs::api_error(MXS_ELAUNCH, msg);
  }
  return decode_step(step, ws, (size_t)MXS_NOALLOC_SCRATCH_BYTES, stream);
}
