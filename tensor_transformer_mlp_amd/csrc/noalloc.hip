// Device scratch of tp_mlp_shard_forward_noalloc: the one entry point that
// allocates no memory (for callers that cannot call hipMalloc: code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The buffer is a file-scope device array of TP_NOALLOC_SCRATCH_BYTES.  Every
// GPU the entry point runs on holds its own copy, at its own address, from
// its first call there (the HIP runtime loads this file's device code, which
// holds the array, when its address is first asked for) until the process
// ends.  In host code the array's name is only a host-side stand-in for the
// symbol, not a device address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept here, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>

#include "tp_mlp.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Address of device `dev`'s copy of the array, looked up with that device
// current (the caller's current device is restored afterwards).
hipError_t lookup(int dev, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) {
    const hipError_t r = hipSetDevice(cur);
    if (e == hipSuccess) e = r;
  }
  if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
  if (e == hipSuccess) *out = p;
  return e;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if ((e = lookup(dev, &p)) != hipSuccess) return e;
    // Two threads may both look it up the first time; they find the same address.
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace tpmlp
