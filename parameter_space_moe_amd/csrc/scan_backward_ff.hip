// Instantiations of the mixed scan's backward for x/dt_raw/B/C in float and dL/dy in float.
#include "scan_backward.hpp"

namespace swimba {
int launch_backward_ff(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws,
                       hipStream_t st) {
  return bwd::launch_bwd_k<float, float>(g, pl, ws, st);
}
}  // namespace swimba
