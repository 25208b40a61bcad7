// Dispatch of the separate design over (input dtype, output dtype).
// Kernels: scan_separate.hpp.
#include "swimba_internal.hpp"

namespace swimba {

int launch_sep_ff(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t, bool);
int launch_sep_fb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t, bool);
int launch_sep_bf(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t, bool);
int launch_sep_bb(const swimba_scan_args*, const ScanPlan&, void*, hipStream_t, bool);

int launch_scan_separate(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st,
                         bool all) {
  const bool in_bf = a->in_dtype == SWIMBA_BF16, out_bf = a->y_dtype == SWIMBA_BF16;
  if (in_bf && out_bf) return launch_sep_bb(a, pl, ws, st, all);
  if (in_bf) return launch_sep_bf(a, pl, ws, st, all);
  if (out_bf) return launch_sep_fb(a, pl, ws, st, all);
  return launch_sep_ff(a, pl, ws, st, all);
}

}  // namespace swimba
