// Router instantiations: 17 to 64 experts.
#include "route.hpp"

namespace swimba {

int launch_route_bf16_wide(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
         float* gate, hipStream_t s) {
  if (E <= 32) return router::launch_route_t<bf16_t, 32>(x, Wr, T, D, E, k, idx, gate, s);
  return router::launch_route_t<bf16_t, 64>(x, Wr, T, D, E, k, idx, gate, s);
}

int launch_route_f32_wide(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
         float* gate, hipStream_t s) {
  if (E <= 32) return router::launch_route_t<float, 32>(x, Wr, T, D, E, k, idx, gate, s);
  return router::launch_route_t<float, 64>(x, Wr, T, D, E, k, idx, gate, s);
}

}  // namespace swimba
