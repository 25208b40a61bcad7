// Instantiations of the mixed scan for x/dt_raw/B/C in float and y in bf16_t.
#include "scan_mixed.hpp"

namespace swimba {
int launch_scan_fb(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return mixed::launch_mixed_w<float, bf16_t>(a, pl, ws, st);
}
}  // namespace swimba
