// Matrix-core sweeps for feature widths padded to 32 (see highd_fwd.h, highd_fwd32.h and
// highd_grad.h).
#include "highd_fwd.h"
#include "highd_fwd32.h"
#include "highd_grad.h"

namespace keops {
namespace hd {
template hipError_t fwd_launch<_Float16, 32>(const FwdArgs&);
template hipError_t fwd_launch<__bf16, 32>(const FwdArgs&);
template hipError_t fwd_launch<float, 32>(const FwdArgs&);
template hipError_t grad_launch<32>(const GradArgs&);
template hipError_t fwd32_launch<_Float16>(const FwdArgs&);
template hipError_t fwd32_launch<__bf16>(const FwdArgs&);
}  // namespace hd
}  // namespace keops
