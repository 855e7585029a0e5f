// The library's own decode workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops that forbid
// allocation): a file-scope device array per GPU, so that
// pkv_paged_attention_decode_noalloc needs no workspace argument.
//
// In host code the array's name is a host-side stand-in, not a device
// address: the address each device holds the array at comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

// Counters first (kStaticCounterSlots int32), then the partial states.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;
};

std::mutex g_mutex;
DeviceScratch g_devices[kMaxDevices];

// Zero n 32-bit words at p (a fill kernel rather than a memset, so the
// clearing is an ordinary kernel node if the first call is captured).
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t static_workspace(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch& d = g_devices[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // the counters must start at zero; every call leaves them zero again
    hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p), kStaticCounterSlots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    d.ptr = p;
  }
  *ptr = d.ptr;
  return hipSuccess;
}

}  // namespace pkv
