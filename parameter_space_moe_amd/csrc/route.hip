// Router dispatch over the x dtype and the expert count.  Kernel: route.hpp.
#include "swimba_internal.hpp"

namespace swimba {

#define SWIMBA_ROUTE_DECL(name)                                                               \
  int name(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,     \
           float* gate, hipStream_t s);
SWIMBA_ROUTE_DECL(launch_route_bf16)
SWIMBA_ROUTE_DECL(launch_route_f32)
SWIMBA_ROUTE_DECL(launch_route_bf16_wide)
SWIMBA_ROUTE_DECL(launch_route_f32_wide)
#undef SWIMBA_ROUTE_DECL

int launch_route(const void* x, swimba_dtype xd, const float* Wr, int64_t T, int D, int E, int k,
                 int32_t* idx, float* gate, hipStream_t s) {
  if (T == 0) return SWIMBA_OK;
  if (xd == SWIMBA_BF16)
    return E <= 16 ? launch_route_bf16(x, Wr, T, D, E, k, idx, gate, s)
                   : launch_route_bf16_wide(x, Wr, T, D, E, k, idx, gate, s);
  return E <= 16 ? launch_route_f32(x, Wr, T, D, E, k, idx, gate, s)
                 : launch_route_f32_wide(x, Wr, T, D, E, k, idx, gate, s);
}

}  // namespace swimba
