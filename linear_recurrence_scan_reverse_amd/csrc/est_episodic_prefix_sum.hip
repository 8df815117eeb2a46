// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<EpisodicPrefixSum>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<EpisodicPrefixSum, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<EpisodicPrefixSum, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EpisodicPrefixSum, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EpisodicPrefixSum, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<EpisodicPrefixSum, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
