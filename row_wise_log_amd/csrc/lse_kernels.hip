// lse_kernels.hip - the entry of the row kernels' launch dispatch: picks the
// element type's instances, which are built in lse_kernels_f32.hip,
// lse_kernels_bf16.hip and lse_kernels_f16.hip.
#include "lse_kernels.h"

namespace lse {

extern template hipError_t launch_dtype<DType::F32>(const LaunchArgs& a);
extern template hipError_t launch_dtype<DType::BF16>(const LaunchArgs& a);
extern template hipError_t launch_dtype<DType::F16>(const LaunchArgs& a);

hipError_t launch(const LaunchArgs& a) {
    if (a.grid <= 0) return hipSuccess;
    switch (a.dtype) {
        case LSE_DTYPE_F32: return launch_dtype<DType::F32>(a);
        case LSE_DTYPE_BF16: return launch_dtype<DType::BF16>(a);
        case LSE_DTYPE_F16: return launch_dtype<DType::F16>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace lse
