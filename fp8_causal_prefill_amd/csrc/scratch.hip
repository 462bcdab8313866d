// Device-resident scratch space for the entry point that may not allocate
// (zyfa_attn_decode_fp8_paged_noalloc): a file-scope array that every GPU the library runs
// on holds from the module's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (with that device current) through hipGetSymbolAddress and
// kept per device; only that address is ever passed to kernels. A call takes the array of
// the device its stream belongs to.
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

hipError_t scratch_of_stream_device(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;  // the null stream belongs to the current device
  if (stream != nullptr) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev, cur] {
    // the array's address on `dev`, looked up with `dev` current (then the caller's
    // current device is restored)
    hipError_t err = dev == cur ? hipSuccess : hipSetDevice(dev);
    void* p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (err == hipSuccess) err = r;
    }
    g_scratch_err[dev] = err;
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace zyfa
