// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<EligibilityTrace>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<EligibilityTrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<EligibilityTrace, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EligibilityTrace, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EligibilityTrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EligibilityTrace, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
