// The fixed device scratch of paged_attn_decode_noalloc, the decode entry
// point for callers that cannot allocate (code under graph capture, tight
// serving loops): its split partial results live in this file-scope device
// array instead of caller-provided workspace.  Each GPU the library runs on
// holds its own copy, at its own address, until the process ends; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device (the array's name is a host-side stand-in, not a device
// address).  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace pa {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // per device, set on its first use

}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -3;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    // with the device current: its own copy of the array
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -3;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return 0;
}

}  // namespace pa
