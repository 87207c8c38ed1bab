// Implicit GEMM with channel-last halo boxes (fp16, MFMA): not built yet.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fc {

bool igemm_halo_fits(const ConvParams&, int32_t, int32_t&, int32_t&, size_t&) { return false; }

int launch_igemm_halo(const Geometry&, const Plan&, const RunArgs&) {
  return FUSEDCONV_ERR_ROUTE;
}

}  // namespace fc
