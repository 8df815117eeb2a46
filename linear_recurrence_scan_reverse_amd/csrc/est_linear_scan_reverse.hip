// Kernel instantiations for one estimator (compiled separately to keep
// build times short; see rlscan_kernel.hpp for the algorithm).
#include "rlscan_launch.hpp"

namespace rlscan {
template hipError_t launch<LinearScanReverse>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<LinearScanReverse, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_typed<LinearScanReverse, F16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanReverse, F32S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanReverse, Bf16S>(const KernelArgs&, hipStream_t);
template hipError_t launch_tm<LinearScanReverse, F16S>(const KernelArgs&, hipStream_t);
}  // namespace rlscan
