// Router instantiations: bf16 x, up to 16 experts.
#include "route.hpp"

namespace swimba {

int launch_route_bf16(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
         float* gate, hipStream_t s) {
  if (E <= 2) return router::launch_route_t<bf16_t, 2>(x, Wr, T, D, E, k, idx, gate, s);
  if (E <= 4) return router::launch_route_t<bf16_t, 4>(x, Wr, T, D, E, k, idx, gate, s);
  if (E <= 8) return router::launch_route_t<bf16_t, 8>(x, Wr, T, D, E, k, idx, gate, s);
  return router::launch_route_t<bf16_t, 16>(x, Wr, T, D, E, k, idx, gate, s);
}

}  // namespace swimba
