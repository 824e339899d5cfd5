// mssm_selective_scan_fwd_noalloc: the scan of mssm_selective_scan_fwd with
// the chunked order's summaries in a fixed device array instead of memory
// the call allocates, for callers that cannot allocate.
//
// `scratch` below is a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  In host code its name is only a
// host-side stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device (with that device current) on
// the first call there, and only that address is ever handed to a kernel.
#include <mutex>

#include "mssm_internal.h"

namespace mssm {

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // MSSM_NOALLOC_SCRATCH_BYTES

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device).
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t scratch_pointer(void** out) { return scratch_on_current_device(out); }

}  // namespace mssm
