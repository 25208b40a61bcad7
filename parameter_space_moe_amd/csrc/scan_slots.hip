// Dispatch of the per-slot separate design over (input dtype, output dtype).
// Kernels: scan_slots.hpp.
#include "swimba_internal.hpp"

namespace swimba {

int launch_slots_ff(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_slots_fb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_slots_bf(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);
int launch_slots_bb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t);

int launch_scan_slots(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  const bool in_bf = a->in_dtype == SWIMBA_BF16, out_bf = a->y_dtype == SWIMBA_BF16;
  if (in_bf && out_bf) return launch_slots_bb(a, pl, ws, st);
  if (in_bf) return launch_slots_bf(a, pl, ws, st);
  if (out_bf) return launch_slots_fb(a, pl, ws, st);
  return launch_slots_ff(a, pl, ws, st);
}

}  // namespace swimba
