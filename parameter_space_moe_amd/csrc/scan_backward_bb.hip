// Instantiations of the mixed scan's backward for x/dt_raw/B/C in bf16_t and dL/dy in bf16_t.
#include "scan_backward.hpp"

namespace swimba {
int launch_backward_bb(const swimba_scan_grad_args* g, const BwdPlan& pl, void* ws,
                       hipStream_t st) {
  return bwd::launch_bwd_k<bf16_t, bf16_t>(g, pl, ws, st);
}
}  // namespace swimba
