// The workspace of pisa_forward_noalloc: a file-scope device array used in place of an attached
// workspace, for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc). Each GPU the library runs on holds its own copy
// of kStaticWorkspaceBytes until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address: its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and kept; only that
// address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pisa_internal.h"

namespace pisa {
namespace {

static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t static_workspace(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace pisa
