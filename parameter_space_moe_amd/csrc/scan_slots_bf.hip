// Instantiations of the per-slot separate design for x/dt_raw/B/C in bf16_t and y in float.
#include "scan_slots.hpp"

namespace swimba {
int launch_slots_bf(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return slots::launch_slots_e<bf16_t, float>(a, pl, ws, st);
}
}  // namespace swimba
