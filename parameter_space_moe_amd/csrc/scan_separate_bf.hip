// Instantiations of the separate design for x/dt_raw/B/C in bf16_t and y in float.
#include "scan_separate.hpp"

namespace swimba {
int launch_sep_bf(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st,
                 bool all) {
  return sep::launch_sep_e<bf16_t, float>(a, pl, ws, st, all);
}
}  // namespace swimba
