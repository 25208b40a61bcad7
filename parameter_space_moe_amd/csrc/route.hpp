// Swimba router for gfx950: logits x . Wr, top-k, softmax over the selected
// logits ("Swimba: Switch Mamba Model Scales State Space Models", Dutch summary
// "Kernmechanisme van Swimba": a router gives each token weights over the
// active experts, top-1 or top-k).
//
// Mapping.  A wave owns R = 64 / EC tokens (EC = E rounded up to a power of
// two).  Per step, lane l reads channels [s*256 + 4l, s*256 + 4l + 4) of each
// of its R token rows -- contiguous across the wave, straight from HBM into
// VGPRs -- and the matching 4 rows of Wr (L2-resident), and accumulates R x EC
// partial logits.  A transpose-reduce across the 64 lanes (6 lane-exchange
// levels, halving the values per lane each time) then leaves lane l holding
// the full logit of (token l / EC, expert l % EC).  The top k of a token are
// picked by a tournament among its EC lanes.
//
// Rounding.  Each lane sums its D/64 channels in the workgroup's step order,
// then the 6 levels add pairs, so the fp32 logit differs from the exact sum by
// at most
// gamma_m * sum_d |x_d Wr[d,e]| with m = ceil(D / 64) + 6,
// gamma_m = m u / (1 - m u), u = 2^-24.
#pragma once
#include <type_traits>

#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace router {

constexpr int kRouteThreads = 256;
constexpr int kCPL = 4;  // channels per lane per step

// Raw 4 consecutive channels of x.  VEC: one 8- or 16-byte load.  Loads are
// unconditional from a clamped (valid) address -- a load under a branch would
// be waited on inside that branch -- and masked when converted.
template <typename TIn, bool VEC>
struct Raw4 {
  using V = typename std::conditional<sizeof(TIn) == 2, uint2, float4>::type;
  V v;
  TIn s[kCPL];
};

template <typename TIn, bool VEC>
__device__ __forceinline__ void load4(const TIn* row, int d, int D, bool ok, Raw4<TIn, VEC>& r) {
  if (VEC) {
    r.v = *reinterpret_cast<const typename Raw4<TIn, VEC>::V*>(row + (ok ? d : 0));
  } else {
#pragma unroll
    for (int c = 0; c < kCPL; ++c) r.s[c] = row[min(ok ? d + c : 0, D - 1)];
  }
}

// MASK: the step may run past D (its last step); otherwise every lane's four
// channels exist and no select is needed.
template <typename TIn, bool VEC, bool MASK = true>
__device__ __forceinline__ void cvt4(const Raw4<TIn, VEC>& r, int d, int D, bool ok, float* v) {
  if (VEC) {
    if constexpr (sizeof(TIn) == 2) {
      v[0] = __uint_as_float(r.v.x << 16);
      v[1] = __uint_as_float(r.v.x & 0xffff0000u);
      v[2] = __uint_as_float(r.v.y << 16);
      v[3] = __uint_as_float(r.v.y & 0xffff0000u);
    } else {
      v[0] = r.v.x;
      v[1] = r.v.y;
      v[2] = r.v.z;
      v[3] = r.v.w;
    }
    if constexpr (MASK) {
#pragma unroll
      for (int c = 0; c < kCPL; ++c) v[c] = ok ? v[c] : 0.f;
    }
  } else {
#pragma unroll
    for (int c = 0; c < kCPL; ++c) v[c] = (ok && d + c < D) ? to_f32(r.s[c]) : 0.f;
  }
}

// Wr rows of one 256-channel step in LDS, shared by the workgroup's four
// waves (each owns different tokens): element (channel 4l + c, expert 4qe..)
// sits at float4 index (c * EC/4 + qe) * kRow + l, so lane l's reads of its
// four rows are contiguous across the wave.  Rows are padded to kRow = 65
// float4s: the staging stores, where consecutive lanes write consecutive
// rows, then fall on different banks.
constexpr int kRow = 65;
template <int EC>
struct WStage {
  static_assert(EC >= 4 && EC % 4 == 0, "experts are staged as float4s");
  static constexpr int kVecs = 64 * kCPL * EC / 4;                  // float4s per step
  static constexpr int kPerThread = (kVecs + kRouteThreads - 1) / kRouteThreads;
  static constexpr int kSlots = kCPL * EC / 4 * kRow;               // LDS float4s per step
  float4 v[kPerThread];
};

template <int EC, bool EXACT>
__device__ __forceinline__ void wstage_load(const float* Wr, int D, int E, int dc, int tid,
                                            WStage<EC>& st) {
#pragma unroll
  for (int j = 0; j < WStage<EC>::kPerThread; ++j) {
    const int i = tid + kRouteThreads * j;
    const int ch = i / (EC / 4), qe = i % (EC / 4);
    const int d = dc + ch;
    const int row = d < D ? d : D - 1;
    const float* w = Wr + (size_t)row * E;
    float4 v;
    if (EXACT) {
      v = *reinterpret_cast<const float4*>(w + qe * 4);
    } else {
      v = make_float4(w[min(qe * 4 + 0, E - 1)], w[min(qe * 4 + 1, E - 1)],
                      w[min(qe * 4 + 2, E - 1)], w[min(qe * 4 + 3, E - 1)]);
    }
    const bool ok = i < WStage<EC>::kVecs && d < D;
    st.v[j] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int EC>
__device__ __forceinline__ void wstage_store(float4* buf, int tid, const WStage<EC>& st) {
#pragma unroll
  for (int j = 0; j < WStage<EC>::kPerThread; ++j) {
    const int i = tid + kRouteThreads * j;
    if (i < WStage<EC>::kVecs) {
      const int ch = i / (EC / 4), qe = i % (EC / 4);
      const int l = ch / kCPL, c = ch % kCPL;
      buf[(c * (EC / 4) + qe) * kRow + l] = st.v[j];
    }
  }
}

// EXACT: E == EC (no padded experts).  VEC: D is a multiple of 4 and x is
// aligned for 4-channel vector loads.  WLDS: Wr steps are staged in LDS and
// shared by the workgroup's waves (4 <= EC <= 16).
template <typename TIn, int EC, bool EXACT, bool VEC, bool WLDS>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const TIn* __restrict__ x,
                                                             const float* __restrict__ Wr,
                                                             int64_t T, int D, int E, int k,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ gate) {
  constexpr int R = 64 / EC;  // tokens per wave
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kRouteThreads / 64) +
                       uniform((int)(threadIdx.x >> 6));
  const int64_t t0 = wave * R;
  // waves past the last token still take part in the staging barriers
  if (!WLDS && t0 >= T) return;
  const bool live = t0 < T;

  // partial logits acc[r * EC + e]
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;

  const TIn* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = x + (t0 + r < T ? t0 + r : T - 1) * D;
  (void)live;

  // Steps of 256 channels, visited from a per-workgroup starting step: every
  // workgroup reads all of Wr, and staggered starts spread those reads over
  // the L2 channels instead of sending all compute units to the same lines.
  constexpr int kStep = 64 * kCPL;
  const int nsteps = (D + kStep - 1) / kStep;
  const int s0 = (int)(blockIdx.x % (unsigned)nsteps);
  auto step_base = [&](int i) {
    const int st = s0 + i;
    return (st >= nsteps ? st - nsteps : st) * kStep;
  };

  // x rows of the next step are in flight while the current step computes
  Raw4<TIn, VEC> xn[R];
  {
    const int d = step_base(0) + lane * kCPL;
#pragma unroll
    for (int r = 0; r < R; ++r) load4<TIn, VEC>(rows[r], d, D, d < D, xn[r]);
  }
  if constexpr (WLDS) {
    __shared__ float4 wbuf[2][WStage<EC>::kSlots];
    const int tid = threadIdx.x;
    WStage<EC> st;
    wstage_load<EC, EXACT>(Wr, D, E, step_base(0), tid, st);
    wstage_store<EC>(wbuf[0], tid, st);
    __syncthreads();
    int buf = 0;
    for (int i = 0; i < nsteps; ++i, buf ^= 1) {
      const int d = step_base(i) + lane * kCPL;
      const bool ok = d < D;
      const bool more = i + 1 < nsteps;
      float xv[R][kCPL];
      if (step_base(i) + kStep <= D) {  // a whole step (uniform): no masking
#pragma unroll
        for (int r = 0; r < R; ++r) cvt4<TIn, VEC, false>(xn[r], d, D, ok, xv[r]);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) cvt4<TIn, VEC, true>(xn[r], d, D, ok, xv[r]);
      }
      if (more) {
        // the stage first: waiting for it below leaves the x loads in flight
        const int dcn = step_base(i + 1), dn = dcn + lane * kCPL;
        wstage_load<EC, EXACT>(Wr, D, E, dcn, tid, st);
#pragma unroll
        for (int r = 0; r < R; ++r) load4<TIn, VEC>(rows[r], dn, D, dn < D, xn[r]);
      }
#pragma unroll
      for (int c = 0; c < kCPL; ++c) {
        float w[EC];
#pragma unroll
        for (int qe = 0; qe < EC / 4; ++qe) {
          const float4 v = wbuf[buf][(c * (EC / 4) + qe) * kRow + lane];
          w[4 * qe + 0] = v.x;
          w[4 * qe + 1] = v.y;
          w[4 * qe + 2] = v.z;
          w[4 * qe + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < EC; ++e) acc[r * EC + e] = fmaf(xv[r][c], w[e], acc[r * EC + e]);
      }
      if (more) wstage_store<EC>(wbuf[buf ^ 1], tid, st);
      __syncthreads();
    }
  } else {
    for (int i = 0; i < nsteps; ++i) {
      const int d = step_base(i) + lane * kCPL;
      const bool ok = d < D;
      float xv[R][kCPL];
#pragma unroll
      for (int r = 0; r < R; ++r) cvt4<TIn, VEC>(xn[r], d, D, ok, xv[r]);
      const int dn = step_base(i + 1 < nsteps ? i + 1 : i) + lane * kCPL;
      if (i + 1 < nsteps) {
#pragma unroll
        for (int r = 0; r < R; ++r) load4<TIn, VEC>(rows[r], dn, D, dn < D, xn[r]);
      }
      // Wr rows of this lane's channels.  Lanes past D (x = 0 there) and padded
      // experts (lanes e >= E, never reported) read clamped, valid rows/columns.
      float w[kCPL][EC];
#pragma unroll
      for (int c = 0; c < kCPL; ++c) {
        const int row = ok ? (VEC ? d + c : min(d + c, D - 1)) : 0;
        const float* wr = Wr + (size_t)row * E;
#pragma unroll
        for (int e = 0; e < EC; ++e) w[c][e] = wr[EXACT ? e : min(e, E - 1)];
      }
#pragma unroll
      for (int c = 0; c < kCPL; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < EC; ++e)
            acc[r * EC + e] = fmaf(xv[r][c], w[c][e], acc[r * EC + e]);
    }
  }

  // transpose-reduce: at level m (32, 16, ..., 1) a lane keeps the half of its
  // values selected by its bit m and adds its partner's copy of that half; at
  // the end lane l holds the full sum of value l.  Levels 32 and 16 use the
  // lane swap instructions (xchg_add), the others DPP permutes (xor_lane).
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = xchg_add<32>(acc[i], acc[i + 32]);
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = xchg_add<16>(acc[i], acc[i + 16]);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const float send = hi ? acc[i] : acc[i + m];
      const float keep = hi ? acc[i + m] : acc[i];
      acc[i] = keep + xor_lane_any(send, m, lane);
    }
  }
  const int r = lane / EC, e = lane % EC;
  const int64_t t = t0 + r;
  float v = acc[0];
  const bool real = e < E;

  // top-k among the EC lanes of token r: (logit desc, expert asc)
  bool taken = false;
  float m0 = 0.f, z = 0.f;
  float my_sel = 0.f;  // logit of the slot this lane reports (lane e reports slot e)
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    bool cand = real && !taken;
    float bv = v;
    int be = e;
#pragma unroll
    for (int o = 1; o < EC; o <<= 1) {
      const float ov = xor_lane_any(bv, o, lane);
      const int oe = xor_lane_any(be, o, lane);
      const bool oc = xor_lane_any((int)cand, o, lane) != 0;
      // the lower expert index wins unless the higher one is strictly larger
      bool take_other;
      if (!cand)
        take_other = oc;
      else if (!oc)
        take_other = false;
      else if (oe < be)
        take_other = !(bv > ov);
      else
        take_other = ov > bv;
      if (take_other) {
        bv = ov;
        be = oe;
        cand = true;
      }
    }
    if (e == be) taken = true;
    if (j == 0) m0 = bv;
    if (e == j) {
      my_sel = bv;
      my_idx = be;
    }
    z += hw_exp2((bv - m0) * kLog2e);
  }
  if (live && t < T && e < k) {
    idx[t * k + e] = my_idx;
    gate[t * k + e] = hw_exp2((my_sel - m0) * kLog2e) / z;
  }
}

template <typename TIn, int EC>
int launch_route_t(const void* x, const float* Wr, int64_t T, int D, int E, int k, int32_t* idx,
                   float* gate, hipStream_t s) {
  constexpr int R = 64 / EC;
  const int64_t waves = (T + R - 1) / R;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(kRouteThreads);
  const size_t vec_bytes = sizeof(TIn) * kCPL;
  const bool vec = ((size_t)D * sizeof(TIn)) % vec_bytes == 0 &&
                   reinterpret_cast<uintptr_t>(x) % vec_bytes == 0;
  const TIn* xp = static_cast<const TIn*>(x);
  const bool exact = E == EC;
  constexpr bool W = EC >= 4 && EC <= 16;  // whole float4s of experts, LDS-sized
  if (vec && exact)
    hipLaunchKernelGGL((route_kernel<TIn, EC, true, true, W>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  else if (vec)
    hipLaunchKernelGGL((route_kernel<TIn, EC, false, true, W>), grid, block, 0, s, xp, Wr, T, D,
                       E, k, idx, gate);
  else if (exact)
    hipLaunchKernelGGL((route_kernel<TIn, EC, true, false, W>), grid, block, 0, s, xp, Wr, T, D,
                       E, k, idx, gate);
  else
    hipLaunchKernelGGL((route_kernel<TIn, EC, false, false, W>), grid, block, 0, s, xp, Wr, T, D,
                       E, k, idx, gate);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

}  // namespace router
}  // namespace swimba
