// noalloc.hip -- the fixed device scratch of the allocation-free forward entry
// point (clear_attn_fwd_noalloc).
//
// One static device array per GPU holds everything that entry point would
// otherwise allocate: the tile map it builds on every call and the text-row
// partials.  Each device the library runs on holds its own copy from the
// moment the code object is loaded there until the process ends.  In host code
// the array's name is only a stand-in: its device address on the current
// device comes from hipGetSymbolAddress, looked up once per device (with that
// device current) and kept; host code passes that address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "clear_internal.h"

static __device__ __align__(256) char scratch[CLEAR_NOALLOC_SCRATCH_BYTES];

namespace clear {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

int noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(CLEAR_ENOTSUP, "device %d: the no-alloc scratch is kept for devices 0..%d", dev,
                     kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(CLEAR_EHIP, "hipGetSymbolAddress (no-alloc scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CLEAR_OK;
}

}  // namespace clear
