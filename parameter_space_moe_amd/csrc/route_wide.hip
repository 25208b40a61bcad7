// Router instantiations: 17 to 64 experts (kernel: route_wide.hpp).
#include "route_wide.hpp"

namespace swimba {

int launch_route_bf16_wide(const void* x, const float* Wr, int64_t T, int D, int E, int k,
                           int32_t* idx, float* gate, hipStream_t s) {
  return router::launch_route_wide_t<bf16_t>(x, Wr, T, D, E, k, idx, gate, s);
}

int launch_route_f32_wide(const void* x, const float* Wr, int64_t T, int D, int E, int k,
                          int32_t* idx, float* gate, hipStream_t s) {
  return router::launch_route_wide_t<float>(x, Wr, T, D, E, k, idx, gate, s);
}

}  // namespace swimba
