// Instantiations of the mixed scan for x/dt_raw/B/C in float and y in float.
#include "scan_mixed.hpp"

namespace swimba {
int launch_scan_ff(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return mixed::launch_mixed_w<float, float>(a, pl, ws, st);
}
}  // namespace swimba
