// Two-output pass: discounted return and TD(lambda) return sharing every load.
#include "rlscan_launch.hpp"

namespace rlscan {

hipError_t launch_returns_td_lambda(const KernelArgs& in, hipStream_t s) {
  const KernelArgs a = resolve_optional(in);
  const int team = stream_team(a);
  switch ((team != 0 && prefer_stream<ReturnsTdLambda>(a, team)) ? team : 0) {
    case 16: return launch_stream<ReturnsTdLambda, 16>(a, s);
    case 32: return launch_stream<ReturnsTdLambda, 32>(a, s);
    case 64: return launch_stream<ReturnsTdLambda, 64>(a, s);
    default: break;
  }
  // rows the streaming kernel does not take: the two single-output kernels
  KernelArgs dr = in;
  dr.v = nullptr;
  dr.out1 = nullptr;
  const hipError_t e = launch<DiscountedReturn>(dr, s);
  if (e != hipSuccess) return e;
  KernelArgs td = in;
  td.out0 = in.out1;
  td.out1 = nullptr;
  return launch<TdLambda>(td, s);
}

}  // namespace rlscan
