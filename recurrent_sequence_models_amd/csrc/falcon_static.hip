// Device scratch of falcon_chunk_fwd_static: the two-kernel chunk-parallel
// path's workspace (per-system key-side images and the carried-state copies)
// held in a fixed array of this library, so that callers which cannot allocate
// device memory can still run that path.
//
// The array below is a device symbol.  In host code its name is only a stand-in,
// not a device address: the address of a device's copy is looked up with
// hipGetSymbolAddress, once per device with that device current, and kept; the
// kernels receive that address as their workspace argument.
#include <hip/hip_runtime.h>

#include <mutex>

#include "falcon.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FALCON_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

namespace falcon {

// Device address of the current device's copy of the scratch array, looked up on
// the first call on that device (a failed lookup is kept and returned again).
hipError_t static_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace falcon
