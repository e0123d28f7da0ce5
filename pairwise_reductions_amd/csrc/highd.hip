// Matrix-core (fp16 / bf16) batched Gauss sum. Not built yet: every shape is reported as
// unsupported so the ABI returns KEOPS_ERR_UNSUPPORTED before launching anything.
#include "internal.h"

namespace keops {

bool highd_supported(int D, int C) {
  (void)D;
  (void)C;
  return false;
}

size_t highd_workspace_bytes(int64_t, int64_t, int64_t, int, int) { return 0; }

hipError_t launch_gauss_sum_highd(const void*, const void*, const void*, float*, void*, int64_t, int64_t,
                                  int64_t, int, int, float, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace keops
