// Device-side helpers shared by the Swimba kernels (gfx950 / CDNA4).
//
// Transcendentals use the hardware's own base-2 instructions (v_exp_f32,
// v_log_f32, about 1 ulp); natural-base constants are folded in by the
// callers so that every exponential in a hot loop is a single v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swimba {

constexpr int kN = 16;          // state entries per channel (the only size built)
constexpr int kWave = 64;       // CDNA wavefront
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

using bf16_t = uint16_t;        // raw bfloat16 bits

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// softplus(z) = max(z, 0) + log1p(exp(-|z|)).  With u = 1 + e rounded,
// 1 + e = u - c where c = (u - 1) - e is the rounding error of u, computed
// exactly; log1p(e) = ln(u - c) = ln(u) - c/u, and ln(u) - c is within
// |c| e of it.  So the result keeps full relative accuracy also for e << 1,
// where ln(u) alone would keep only the bits of e that survive the add (and
// for e below half an ulp of 1 it returns e itself).
__device__ __forceinline__ float softplus_f32(float z) {
  const float e = hw_exp2(-fabsf(z) * kLog2e);
  const float u = 1.0f + e;
  const float l = fmaf(hw_log2(u), kLn2, e - (u - 1.0f));
  return fmaxf(z, 0.0f) + l;
}

// Zero-order-hold factor phi = (exp(z) - 1) / z of the decay a = exp(z) =
// exp2(m): the zero-order-hold input term is phi times the Euler term
// Delta B x.  For a >= 1/2 it is (a - 1) / ln(a) with the computed log of a,
// so that the rounding of a cancels between numerator and denominator
// (Kahan's expm1 method, as given in Goldberg, "What every computer scientist
// should know about floating-point arithmetic"); below 1/2 there is no
// cancellation and z itself divides; phi = 1 when a rounds to 1.
__device__ __forceinline__ float zoh_phi(float a, float m) {
  const float lg = a < 0.5f ? m : hw_log2(a);
  return lg == 0.f ? 1.f : (a - 1.f) * __builtin_amdgcn_rcpf(lg) * kLog2e;
}

// Cross-lane exchanges at lane distance M = 32 or 16 on gfx950's lane-half
// and row swap instructions (VALU, no LDS round trip).  permlane32_swap(x, y)
// exchanges the upper 32 lanes of x with the lower 32 lanes of y;
// permlane16_swap(x, y) exchanges the odd 16-lane rows of x with the even
// rows of y.
template <int M>
__device__ __forceinline__ void lane_swap(float x, float y, float& r0, float& r1) {
  static_assert(M == 32 || M == 16, "swap distances are 32 and 16 lanes");
  const uint32_t a = __float_as_uint(x), b = __float_as_uint(y);
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
  }
}

// One transpose-reduce exchange at distance M: a lane whose bit M is clear
// keeps `lo` and sends `hi`, the others keep `hi` and send `lo`; returns
// keep + the partner's sent value (the two swap results hold exactly those
// two values on every lane; the sum is the same in either order).
template <int M>
__device__ __forceinline__ float xchg_add(float lo, float hi) {
  float r0, r1;
  lane_swap<M>(lo, hi, r0, r1);
  return r0 + r1;
}

// The value of lane (lane ^ M) for M = 32 or 16.
template <int M>
__device__ __forceinline__ float partner(float v, int lane) {
  float r0, r1;
  lane_swap<M>(v, v, r0, r1);
  return (lane & M) ? r0 : r1;
}
// A DPP lane permute of v (CTRL: the DPP control code, all rows and banks).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The value of lane (lane ^ M), M a power of two below 64, without an LDS
// round trip: DPP quad permutes for 1 and 2, a half-row mirror followed by a
// quad reverse for 4, a 16-lane row rotate by 8 for 8, the lane swaps for 16
// and 32.
template <int M>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor distance");
  if constexpr (M == 1) return dpp_mov<0xB1>(v);         // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));  // half-mirror, reverse
  else if constexpr (M == 8) return dpp_mov<0x128>(v);   // row_ror:8
  else return partner<M>(v, lane);
}
// The same for a distance known only after unrolling (constant-folded).
__device__ __forceinline__ float xor_lane_any(float v, int m, int lane) {
  switch (m) {
    case 1: return xor_lane<1>(v, lane);
    case 2: return xor_lane<2>(v, lane);
    case 4: return xor_lane<4>(v, lane);
    case 8: return xor_lane<8>(v, lane);
    case 16: return xor_lane<16>(v, lane);
    default: return xor_lane<32>(v, lane);
  }
}
__device__ __forceinline__ int xor_lane_any(int v, int m, int lane) {
  return __float_as_int(xor_lane_any(__int_as_float(v), m, lane));
}

// Sum over the 64 lanes of a wave, the same on every lane.
__device__ __forceinline__ float wave_sum64(float v) {
  v = xchg_add<32>(v, v);
  v = xchg_add<16>(v, v);
  v += xor_lane<8>(v, 0);
  v += xor_lane<4>(v, 0);
  v += xor_lane<2>(v, 0);
  v += xor_lane<1>(v, 0);
  return v;
}

// Element `i` of a wave-uniform base with a 32-bit byte offset: lets the
// backend address it as SGPR base + unsigned VGPR offset (no 64-bit math).
template <typename T>
__device__ __forceinline__ const T& at32(const T* base, uint32_t i) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + i * (uint32_t)sizeof(T));
}
template <typename T>
__device__ __forceinline__ T& at32(T* base, uint32_t i) {
  return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + i * (uint32_t)sizeof(T));
}

// Non-temporal loads: they do not allocate in the per-CU vector cache.  Used
// where every CU streams the same L2-resident table once (the decode step's
// router), which the cache's miss handling would otherwise throttle.
typedef float f4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f4v_t v = __builtin_nontemporal_load(reinterpret_cast<const f4v_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float load_nt(const float* p) { return __builtin_nontemporal_load(p); }

// Wave-uniform value into an SGPR (the argument must already be uniform).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

}  // namespace swimba
