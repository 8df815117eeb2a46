// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<Vtrace>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Vtrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Vtrace, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Vtrace, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Vtrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Vtrace, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
