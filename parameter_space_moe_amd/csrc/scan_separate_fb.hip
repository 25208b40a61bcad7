// Instantiations of the separate design for x/dt_raw/B/C in float and y in bf16_t.
#include "scan_separate.hpp"

namespace swimba {
int launch_sep_fb(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st,
                 bool all) {
  return sep::launch_sep_e<float, bf16_t>(a, pl, ws, st, all);
}
}  // namespace swimba
