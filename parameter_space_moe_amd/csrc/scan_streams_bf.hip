// Instantiations of the stream-mixed scan for X/dt_raw/B/C in bf16_t and y in float.
#include "scan_streams.hpp"

namespace swimba {
int launch_streams_bf(const swimba_stream_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return streams::launch_streams_k<bf16_t, float>(a, pl, ws, st);
}
}  // namespace swimba
