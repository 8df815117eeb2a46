// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<Gae>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Gae, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Gae, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Gae, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Gae, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Gae, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
