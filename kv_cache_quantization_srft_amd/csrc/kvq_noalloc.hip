// Allocation-free decode: the workspace of kvq_decode_attn (completion counters and chunk
// partials) lives in a file-scope device array, so kvq_decode_attn_noalloc needs no caller
// buffer beyond its inputs and outputs and makes no allocation of any kind.
//
// Every GPU the library runs on holds its own copy of `scratch` (kScratchBytes) until the process
// ends.  Host code never passes the array's name to a kernel: on the first call on a device,
// with that device current, hipGetSymbolAddress resolves the device address of that GPU's copy,
// which is kept per device and used from then on.  The same first call clears the completion
// counters with a fill kernel on the caller's stream; afterwards every call that runs to
// completion leaves them zero (the last work-group of a unit resets its counter).  All calls on
// one GPU share the array: calls that overlap in time on one GPU race.
#include <mutex>

#include "kvq_internal.h"

namespace kvq_impl {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       int(kDecodeCounterBytes / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace kvq_impl
