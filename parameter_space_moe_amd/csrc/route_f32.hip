// Router instantiations: fp32 x, up to 16 experts.
#include "route.hpp"

namespace swimba {

int launch_route_f32(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
         float* gate, hipStream_t s) {
  if (E <= 2) return router::launch_route_t<float, 2>(x, Wr, T, D, E, k, idx, gate, s);
  if (E <= 4) return router::launch_route_t<float, 4>(x, Wr, T, D, E, k, idx, gate, s);
  if (E <= 8) return router::launch_route_t<float, 8>(x, Wr, T, D, E, k, idx, gate, s);
  return router::launch_route_t<float, 16>(x, Wr, T, D, E, k, idx, gate, s);
}

}  // namespace swimba
