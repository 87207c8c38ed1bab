// fusedconv_run_noalloc: fusedconv_run for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc).  The workspace a plan needs (repacked weights, K-split
// partials) lives in `scratch`, a fixed array of this library on each GPU,
// instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"

namespace fc {
namespace {

// One copy per GPU, held until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory): it uses the device address hipGetSymbolAddress returns, kept per
// device below.
static __device__ __align__(256) unsigned char scratch[FUSEDCONV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device; NULL = not looked up

// The current device's copy of the array (looked up once per device, with
// that device current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_last_error(FUSEDCONV_ERR_DEVICE, "no current HIP device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_last_error(FUSEDCONV_ERR_LAUNCH, std::string("hipGetSymbolAddress(scratch): ") +
                                                      hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FUSEDCONV_OK;
}

}  // namespace
}  // namespace fc

extern "C" int fusedconv_run_noalloc(const fusedconv_handle* h, const void* x, const void* w,
                                     const void* bias, const void* z, void* y, void* stream) {
  size_t need = 0;
  int rc = fusedconv_workspace_size(h, &need);
  if (rc != FUSEDCONV_OK) return rc;
  if (need > (size_t)FUSEDCONV_NOALLOC_SCRATCH_BYTES)
    return fc::set_last_error(
        FUSEDCONV_ERR_WORKSPACE,
        "the plan needs " + std::to_string(need) + " workspace bytes; fusedconv_run_noalloc holds " +
            std::to_string((size_t)FUSEDCONV_NOALLOC_SCRATCH_BYTES) +
            " (use fusedconv_run with a caller workspace)");
  void* ws = nullptr;
  if (need > 0) {
    rc = fc::scratch_address(&ws);
    if (rc != FUSEDCONV_OK) return rc;
  }
  // every route writes each workspace byte it later reads (weight repacks fill
  // their whole layout, zero padding included; each K slice writes its whole
  // partial), so nothing needs clearing between calls
  return fusedconv_run_ex(h, x, w, bias, z, y, ws, need, 0u, stream);
}
