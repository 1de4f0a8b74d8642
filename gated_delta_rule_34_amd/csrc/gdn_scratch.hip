// gdn_scratch.hip -- the fixed per-GPU scratch array of gdn_fwd_noalloc (include/gdn.h).
//
// One array of GDN_NOALLOC_SCRATCH_BYTES in device memory, which each GPU the library runs on
// holds until the process ends. In host code `scratch` names a host-side stand-in, not a
// device address: its address on the current device comes from hipGetSymbolAddress, looked
// up once per device (with that device current) and kept; kernels receive that pointer as
// their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace gdn
