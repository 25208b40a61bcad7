// Instantiations of the per-slot separate design for x/dt_raw/B/C in float and y in bf16_t.
#include "scan_slots.hpp"

namespace swimba {
int launch_slots_fb(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return slots::launch_slots_e<float, bf16_t>(a, pl, ws, st);
}
}  // namespace swimba
