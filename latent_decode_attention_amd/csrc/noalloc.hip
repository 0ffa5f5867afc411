// noalloc.hip -- the scratch memory of slimkv_decode_attn_noalloc: a
// file-scope device array that stands in for the caller's workspace, so that
// callers who cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid allocation) can still run the attention.
//
// Each device the library runs on holds its own copy of the array until the
// process ends.  Its address is taken once per device with
// hipGetSymbolAddress and kept; host code never uses the array's own name as
// an address (on the host that name is only a stand-in for the symbol).
// Every call on a device shares the device's array, so calls that overlap
// on one device (two streams) race; the per-unit counters the attention
// kernel elects its merging workgroup with are cleared by a small kernel at
// the start of every call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "internal.h"

namespace slimkv {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, uint32_t words) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < words; i += gridDim.x * 256u) p[i] = 0u;
}

std::mutex g_mu;
std::map<int, void*> g_scratch;  // device -> address of its copy of `scratch`

}  // namespace

hipError_t noalloc_scratch(size_t clear_bytes, hipStream_t s, void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
      p = it->second;
    } else {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev] = p;
    }
  }
  const uint32_t words = (uint32_t)((clear_bytes + 3) / 4);
  if (words > 0) {
    const unsigned blocks = std::min<uint32_t>((words + 255) / 256, 1024u);
    hipLaunchKernelGGL(clear_words_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p),
                       words);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace slimkv
