// Swimba router for gfx950: logits x . Wr, top-k, softmax over the selected
// logits ("Swimba: Switch Mamba Model Scales State Space Models", Dutch summary
// "Kernmechanisme van Swimba": a router gives each token weights over the
// active experts, top-1 or top-k).
//
// Mapping.  A workgroup of four waves owns 64 tokens; lane t of every wave is
// token t.  The waves split the channels into 128-byte pieces, interleaved, so
// the four partial sums per token cover disjoint channel sets.  Each wave
// stages its 64 x-rows of a piece through LDS (coalesced 16-byte loads in, one
// conflict-free row per lane out) and multiplies them by Wr rows that are the
// same for every lane, hence read by the scalar unit into SGPR operands: one
// v_fma per (token, channel, expert).
//
// Rounding.  Every 128-byte piece is summed from zero and then added to the
// wave's total; the four wave totals are added in a fixed order.  The fp32
// logit therefore differs from the exact sum by at most
// gamma_{m} * sum_d |x_d Wr[d,e]| with m = (channels per piece) +
// (pieces per wave) + 2, gamma_m = m u / (1 - m u), u = 2^-24.
#pragma once
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace router {

constexpr int kRouteWaves = 4;
constexpr int kRowBytes = 144;  // 128 data bytes + 16 pad: conflict-free row reads

template <typename TIn, int EC, bool EXACT, bool VEC>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(const TIn* __restrict__ x,
                                                                const float* __restrict__ Wr,
                                                                int64_t T, int D, int E, int k,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ gate) {
  constexpr int CH = 128 / sizeof(TIn);  // channels per piece
  constexpr int PER16 = 16 / sizeof(TIn);
  constexpr int kTileBytes = kRouteWaves * 64 * kRowBytes;
  constexpr int kRedBytes = (kRouteWaves - 1) * EC * 64 * 4;
  constexpr int kSmem = kTileBytes > kRedBytes ? kTileBytes : kRedBytes;
  // full unrolling of the piece for the common expert counts only (code size)
  constexpr int kUnroll = EC <= 16 ? 8 : 1;
  __shared__ __align__(16) unsigned char smem[kSmem];

  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  unsigned char* tile = smem + wave * 64 * kRowBytes;
  const int npieces = (D + CH - 1) / CH;

  float acc[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) acc[e] = 0.f;

  for (int pc = wave; pc < npieces; pc += kRouteWaves) {
    const int dc = pc * CH;
    // stage 64 rows x 128 bytes: lane covers (row, 16-byte column) pairs
    if (VEC) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = lane + 64 * i, r = q >> 3, col = q & 7;
        const int64_t t = t0 + r;
        const int dd = dc + col * PER16;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < T && dd < D) v = *reinterpret_cast<const uint4*>(x + t * D + dd);
        *reinterpret_cast<uint4*>(tile + r * kRowBytes + col * 16) = v;
      }
    } else {
      for (int i = 0; i < CH; ++i) {
        const int q = lane + 64 * i, r = q / CH, c = q % CH;
        const int64_t t = t0 + r;
        const int dd = dc + c;
        TIn v = 0;
        if (t < T && dd < D) v = x[t * D + dd];
        *reinterpret_cast<TIn*>(tile + r * kRowBytes + c * sizeof(TIn)) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float part[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) part[e] = 0.f;
    const int cmax = min(CH, D - dc);  // wave-uniform
    const unsigned char* row = tile + lane * kRowBytes;
    if (cmax == CH) {
#pragma unroll kUnroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + i * 16);
        float xv[PER16];
        if (sizeof(TIn) == 2) {
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[2 * j] = __uint_as_float(w4[j] << 16);
            xv[2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
          }
        } else {
          xv[0] = __uint_as_float(v.x);
          xv[1] = __uint_as_float(v.y);
          xv[2] = __uint_as_float(v.z);
          xv[3] = __uint_as_float(v.w);
        }
#pragma unroll
        for (int j = 0; j < PER16; ++j) {
          const float* w = Wr + (size_t)(dc + i * PER16 + j) * E;
#pragma unroll
          for (int e = 0; e < EC; ++e)
            if (EXACT || e < E) part[e] = fmaf(xv[j], w[e], part[e]);
        }
      }
    } else {
      for (int c = 0; c < cmax; ++c) {
        const float xv = to_f32(*reinterpret_cast<const TIn*>(row + c * sizeof(TIn)));
        const float* w = Wr + (size_t)(dc + c) * E;
#pragma unroll
        for (int e = 0; e < EC; ++e)
          if (EXACT || e < E) part[e] = fmaf(xv, w[e], part[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < EC; ++e) acc[e] += part[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // reduce the four wave totals in a fixed order (wave 0 + 1 + 2 + 3)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E) red[((wave - 1) * EC + e) * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
  const int64_t t = t0 + lane;
#pragma unroll
  for (int w = 0; w < kRouteWaves - 1; ++w)
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E) acc[e] += red[(w * EC + e) * 64 + lane];
  if (t >= T) return;

  // top-k by (logit descending, expert ascending).  The selected logits go to
  // LDS column `lane` (each lane has consumed its own column of `red` above,
  // and k <= E rows fit in the buffer).
  float* sel = red;
  uint64_t taken = 0;
  float m = 0.f;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bv = 0.f;
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      if (e < E && !((taken >> e) & 1ull)) {
        if (best < 0 || acc[e] > bv) {
          best = e;
          bv = acc[e];
        }
      }
    }
    taken |= 1ull << best;
    if (j == 0) m = bv;
    idx[t * k + j] = best;
    sel[j * 64 + lane] = bv;
  }
  float z = 0.f;
  for (int j = 0; j < k; ++j) z += hw_exp2((sel[j * 64 + lane] - m) * kLog2e);
  for (int j = 0; j < k; ++j) gate[t * k + j] = hw_exp2((sel[j * 64 + lane] - m) * kLog2e) / z;
}

// EXACT: E == EC, no per-expert guard in the inner loop.
template <typename TIn, int EC>
int launch_route_t(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
                   float* gate, hipStream_t s) {
  const dim3 grid((unsigned)((T + 63) / 64)), block(kRouteWaves * 64);
  const bool vec = ((D * sizeof(TIn)) % 16 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  const TIn* xp = static_cast<const TIn*>(x);
  const bool exact = E == EC;
  if (vec && exact)
    hipLaunchKernelGGL((route_kernel<TIn, EC, true, true>), grid, block, 0, s, xp, Wr, T, D, E, k,
                       idx, gate);
  else if (vec)
    hipLaunchKernelGGL((route_kernel<TIn, EC, false, true>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  else if (exact)
    hipLaunchKernelGGL((route_kernel<TIn, EC, true, false>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  else
    hipLaunchKernelGGL((route_kernel<TIn, EC, false, false>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

}  // namespace router
}  // namespace swimba
