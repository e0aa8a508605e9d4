// na_forward_noalloc: the GNA forward for callers that cannot allocate
// device memory.  Its one scratch buffer -- the tile map the attention
// kernel walks -- lives in a fixed, file-scope device array instead of a
// cached hipMalloc allocation.  Each GPU the library runs on holds its own
// copy of the array until the process ends; every call on that GPU reuses it
// (so calls that overlap on one GPU race: they must be ordered, e.g. on one
// stream).
#include <hip/hip_runtime.h>

#include <mutex>

#include "forward_buffer.hpp"
#include "na.h"

// The buffer itself.  In host code its name is a host-side stand-in, not a
// device address: only the pointer hipGetSymbolAddress returns for it (per
// device) is ever used.
static __device__ __align__(256) unsigned char scratch[NA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" na_status na_forward_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                        int batch, int heads, int head_dim, const int grid[3], const int window[3],
                                        const int stride[3], float scale, na_dtype dtype, void* stream) {
  return na::forward_in_buffer(q, k, v, out, lse, batch, heads, head_dim, grid, window, stride, scale, dtype, stream,
                               NA_NOALLOC_SCRATCH_BYTES, &scratch_address);
}
