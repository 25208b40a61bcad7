// Instantiations of the per-slot separate design for x/dt_raw/B/C in float and y in float.
#include "scan_slots.hpp"

namespace swimba {
int launch_slots_ff(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return slots::launch_slots_e<float, float>(a, pl, ws, st);
}
}  // namespace swimba
