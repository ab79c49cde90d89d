// verify_mfma.hip - bf16 MFMA split-K partial kernel (not yet implemented).
#include "va_internal.h"

namespace va {

hipError_t launch_mfma_partial(const RunArgs &, const Workspace &, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace va
