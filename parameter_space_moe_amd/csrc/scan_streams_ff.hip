// Instantiations of the stream-mixed scan for X/dt_raw/B/C in float and y in float.
#include "scan_streams.hpp"

namespace swimba {
int launch_streams_ff(const swimba_stream_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  return streams::launch_streams_k<float, float>(a, pl, ws, st);
}
}  // namespace swimba
