// Device-resident scratch space for the entry point that may not allocate
// (zyfa_attn_decode_fp8_paged_noalloc): a file-scope array that every GPU the library runs
// on holds from the module's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (with that device current) through hipGetSymbolAddress and
// kept per device; only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace zyfa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
}  // namespace

hipError_t scratch_of_current_device(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace zyfa
