// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<Retrace>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Retrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<Retrace, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Retrace, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Retrace, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<Retrace, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
