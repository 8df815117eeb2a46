// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<DiscountedReturn>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<DiscountedReturn, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<DiscountedReturn, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<DiscountedReturn, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<DiscountedReturn, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<DiscountedReturn, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
