// Fixed device scratch for attn_bwd_noalloc: the backward pass's workspace
// held in a file-scope device array instead of memory the caller allocates.
//
// Each GPU the library runs on holds its own copy of `scratch` (the code
// object's data, allocated when the library's kernels are loaded on that GPU)
// until the process ends. In host code the array's name is only a stand-in
// for the symbol; its device address is looked up once per device with
// hipGetSymbolAddress and that address is what the kernels are given.
#include <mutex>

#include "attn_launch.h"

namespace tam {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace tam
