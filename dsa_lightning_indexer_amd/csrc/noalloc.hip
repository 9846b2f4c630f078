// indexcache_forward without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  The kernels' scratch memory (decode scores, select
// state, attention split partials) lives in one file-scope device array of
// DSA_NOALLOC_SCRATCH_BYTES per GPU, loaded with the library and kept until the
// process ends.  Every call on a GPU uses that GPU's copy, so calls that
// overlap on one GPU race; each kernel sequence clears the state it needs to
// start at zero with its own fill kernels, as it does in a caller workspace.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "common.hpp"

// Device-side storage.  In host code this name is only a stand-in: its device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device); NULL with the error text set on failure.
void* scratch_on_current_device(dsa_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  char msg[256];
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
    *st = dsa_host::set_error(DSA_ERR_HIP, msg);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof(msg), "device %d outside the %d devices the scratch table holds", dev, kMaxDevices);
    *st = dsa_host::set_error(DSA_ERR_UNSUPPORTED, msg);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      *st = dsa_host::set_error(DSA_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

dsa_status indexcache_forward_noalloc(const char* pattern, int32_t n_layers, const dsa_layer* layers, int32_t k,
                                      int32_t* src_layer, hipStream_t stream) {
  // Validation and the scratch need first: nothing touches the device when the
  // arguments are rejected.
  size_t need = 0;
  dsa_status st = dsa_host::forward_workspace_need(pattern, n_layers, layers, k, &need);
  if (st != DSA_OK) return st;
  if (need > kNoAllocScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof(msg), "these layers need %zu bytes of scratch; the allocation-free entry point holds %zu",
             need, kNoAllocScratchBytes);
    return dsa_host::set_error(DSA_ERR_WORKSPACE, msg);
  }
  void* ws = scratch_on_current_device(&st);
  if (!ws) return st;
  return indexcache_forward(pattern, n_layers, layers, k, src_layer, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
