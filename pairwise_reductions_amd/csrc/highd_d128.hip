// Matrix-core sweeps for feature widths padded to 128 (see highd_fwd.h and highd_grad.h).
#include "highd_fwd.h"
#include "highd_grad.h"

namespace keops {
namespace hd {
template hipError_t fwd_launch<_Float16, 128>(const FwdArgs&);
template hipError_t fwd_launch<__bf16, 128>(const FwdArgs&);
template hipError_t fwd_launch<float, 128>(const FwdArgs&);
template hipError_t grad_launch<128>(const GradArgs&);
}  // namespace hd
}  // namespace keops
