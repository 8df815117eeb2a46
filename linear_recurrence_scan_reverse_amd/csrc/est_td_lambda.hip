// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<TdLambda>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<TdLambda, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<TdLambda, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<TdLambda, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<TdLambda, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<TdLambda, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
