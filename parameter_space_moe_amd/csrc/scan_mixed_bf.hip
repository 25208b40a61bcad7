// Instantiations of the mixed scan for x/dt_raw/B/C in bf16_t and y in float.
#include "scan_mixed.hpp"

namespace swimba {
int launch_scan_bf(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return mixed::launch_mixed_w<bf16_t, float>(a, pl, ws, st);
}
}  // namespace swimba
