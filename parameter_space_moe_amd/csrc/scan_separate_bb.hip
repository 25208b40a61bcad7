// Instantiations of the separate design for x/dt_raw/B/C in bf16_t and y in bf16_t.
#include "scan_separate.hpp"

namespace swimba {
int launch_sep_bb(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st,
                 bool all) {
  return sep::launch_sep_e<bf16_t, bf16_t>(a, pl, ws, st, all);
}
}  // namespace swimba
