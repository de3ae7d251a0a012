// Fixed device scratch for the allocation-free forward entry point.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the split-KV
// partials of the few-query head_dim-16 route from this file-scope array
// instead of a workspace argument.  Each GPU holds its own copy of the array
// at its own address until the process ends; the address is looked up once
// per device with hipGetSymbolAddress and kept.  Every call on one GPU shares
// that GPU's array, and the split-KV kernels write every partial they read,
// so nothing needs clearing between calls; calls that overlap on one GPU
// (two streams, two threads) race on it.
#include <mutex>

#include "common.h"

namespace sdpa {
namespace {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // the device is current: its copy of the array is the one looked up
  std::call_once(g_once[dev], [dev] { g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch)); });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sdpa
