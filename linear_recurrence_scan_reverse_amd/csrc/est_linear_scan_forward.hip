// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<LinearScanForward>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<LinearScanForward, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<LinearScanForward, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanForward, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanForward, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanForward, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
