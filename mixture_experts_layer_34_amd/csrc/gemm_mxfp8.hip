// Expert-grouped MXFP8 GEMMs (scaled MFMA) — forward UP and DOWN only.
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"

namespace mok {

hipError_t gemm_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  (void)kind; (void)g; (void)s;
  return hipErrorNotSupported;
}

}  // namespace mok
