// lse_kernels_bf16.hip - the bf16 instances of the row-wise LSE kernels
// (lse_kernels.h), in a translation unit of their own.
#include "lse_kernels.h"

namespace lse {
template hipError_t launch_dtype<DType::BF16>(const LaunchArgs& a);
}  // namespace lse
