// scratch.hip -- the device array behind the entry points that allocate
// nothing (attn_decode_splitkv_noalloc): a file-scope __device__ buffer of
// a fixed size, one copy per GPU for the life of the process.
//
// In host code the name `scratch` stands for a host-side shadow, not a
// device address.  Its device address is looked up once per device, with
// that device current, through hipGetSymbolAddress, and only that address
// is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[rattn::kScratchBytes];

namespace rattn {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace rattn
