// Device scratch for the allocation-free entry point (sta_backward_noalloc).
//
// Some callers cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it). For them the backward's
// per-row workspace D = rowsum(dO * O) lives in a file-scope device array that
// the code object carries: every GPU the library runs on holds its own copy
// from module load until the process ends. Its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and cached;
// host code never passes the array's name itself to a kernel or a copy.
//
// Every call on one GPU shares that GPU's array, and the array keeps the last
// call's contents: calls that overlap on one GPU (two streams, two threads)
// race on it. The backward's delta kernel writes every row of D it later
// reads, so nothing in the array needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sta_kernels.h"

namespace sta {
namespace {

static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

int noalloc_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace sta
