// gdn_host_stubs.cpp -- host-only stand-ins for the kernel launchers and the trace hooks, so
// that the C ABI's host code (gdn_abi.cpp) links into a CPU build under AddressSanitizer and
// UndefinedBehaviorSanitizer. Every launcher returns success without touching a GPU; the
// sanitized build is used only by tests whose calls are all rejected, or sized, on the host.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {
bool trace_on() { return false; }
void trace_launch(const char*, hipStream_t, void (*launch)(const void*), const void* ctx) { launch(ctx); }
hipError_t launch_forward(const Prob&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_backward(const Prob&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_conv(const ConvArgs&, int, bool, hipStream_t) { return hipSuccess; }
void* noalloc_scratch() { return nullptr; }
}  // namespace gdn

extern "C" {
gdn_status gdn_trace_enable(int) { return GDN_OK; }
int gdn_trace_collect(gdn_trace_entry*, int) { return 0; }
}
