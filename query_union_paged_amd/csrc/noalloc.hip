// pw_union_attention_noalloc: pw_union_attention for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The re-tiled K/V copy and page factors, which
// pw_union_attention keeps in the caller's workspace, live here in a
// file-scope device array instead.
//
// Each device holds its own copy of `scratch` at its own address; host code
// never passes the array's name to a kernel (in host code it names a host-side
// stand-in), only the device address that hipGetSymbolAddress returns for the
// current device, looked up once per device on the first call there.  Every
// call on a device reuses that device's array, so calls that overlap on one
// device race; the re-tiling pass rewrites every byte a call reads, so nothing
// needs clearing between calls.
#include <mutex>

#include "pw_internal.h"

namespace {

constexpr size_t kScratchBytes = PW_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];                    // device address per device, once set

}  // namespace

namespace pw {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace pw
