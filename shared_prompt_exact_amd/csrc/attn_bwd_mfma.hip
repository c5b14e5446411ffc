// Backward pass on gfx950 matrix cores (not yet built: the scalar path
// serves every backward until this lands).
#include "mfma_common.h"

namespace dualkv {

bool bwd_mfma_supported(const Problem&) { return false; }
size_t bwd_mfma_workspace_bytes(const Problem&) { return 0; }
hipError_t launch_bwd_mfma(const Problem&, const void*, const void*, const void*, const void*,
                           const float*, const void*, void*, void*, void*, void*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace dualkv
