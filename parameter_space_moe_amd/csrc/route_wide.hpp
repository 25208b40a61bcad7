// Swimba router for 17..64 experts on gfx950: logits x . Wr, top-k, softmax
// over the selected logits ("Swimba: Switch Mamba Model Scales State Space
// Models", Dutch summary "Kernmechanisme van Swimba"; Spanish summary
// "Escalabilidad": more experts in total at a fixed number of active ones).
//
// Mapping.  The 16-expert router's register blocking per wave (4 tokens x 16
// experts, lanes over channels) is kept.  A workgroup has 4 waves: 2 token
// groups x 2 slices of 16 experts, so that two workgroups fit a compute unit
// (one's step barriers overlap the other's arithmetic).  Each 256-channel
// step of Wr for the pass's 32 experts is staged in LDS, double-buffered, and
// read by both token groups; the x rows of a token group are read by its two
// waves (the second read hits the vector cache).  Experts 33..64 take a
// second pass over the channels.  After each pass the waves write their 64
// logits to LDS; one wave per token group then picks each token's top k
// over all E experts: every lane of a token's 16 takes the best of its (up
// to 4) experts, then the 16 lanes hold a tournament.
//
// Rounding is the 16-expert router's: each lane sums its D/64 channels in the
// workgroup's step order, then 6 transpose-reduce levels add pairs.
#pragma once
#include "route.hpp"

namespace swimba {
namespace router {

constexpr int kWideEC = 16;  // experts per wave and pass
constexpr int kWideR = 4;    // tokens per wave
constexpr int kWideTG = 2;   // token groups per workgroup
constexpr int kWideEG = 2;   // 16-expert slices per pass
constexpr int kWidePasses = 2;  // passes over the channels (32 experts each)
constexpr int kSlice = 16 * kRow;  // LDS float4s of one 16-expert slice of a step

struct WideStage {
  static constexpr int kThreads = 64 * kWideTG * kWideEG;
  static constexpr int kVecs = kWideEG * 1024;  // float4s per step: 256 channels x 32 experts
  static constexpr int kPerThread = kVecs / kThreads;
  float4 v[kPerThread];
};

// Wr rows of the step at channel dc for the pass's experts eb..eb+31:
// element (channel 4l + c, expert eb + 16 g + 4 qe ..) sits at float4 index
// g * kSlice + (c * 4 + qe) * kRow + l (rows padded to kRow float4s, so the
// staging stores fall on different banks), so a wave's reads of its slice are
// lane-contiguous.  Experts past E and channels past D read as 0.
// VEC4: E is a multiple of 4 and Wr 16-byte aligned (one 16-byte load per
// four experts).
template <bool VEC4>
__device__ __forceinline__ void wide_stage_load(const float* Wr, int D, int E, int eb, int dc,
                                                int tid, WideStage& st) {
#pragma unroll
  for (int j = 0; j < WideStage::kPerThread; ++j) {
    const int i = tid + WideStage::kThreads * j;
    const int g = i >> 10, r = i & 1023, ch = r >> 2, qe = r & 3;
    const int d = dc + ch;
    const int row = d < D ? d : D - 1;
    const int e0 = eb + g * 16 + qe * 4;
    const float* w = Wr + (size_t)row * E;
    const bool ok = d < D;
    if (VEC4) {
      const float4 v = *reinterpret_cast<const float4*>(w + min(e0, E - 4));
      st.v[j] = ok && e0 < E ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const float v0 = w[min(e0 + 0, E - 1)], v1 = w[min(e0 + 1, E - 1)];
      const float v2 = w[min(e0 + 2, E - 1)], v3 = w[min(e0 + 3, E - 1)];
      st.v[j] = make_float4(ok && e0 + 0 < E ? v0 : 0.f, ok && e0 + 1 < E ? v1 : 0.f,
                            ok && e0 + 2 < E ? v2 : 0.f, ok && e0 + 3 < E ? v3 : 0.f);
    }
  }
}

__device__ __forceinline__ void wide_stage_store(float4* buf, int tid, const WideStage& st) {
#pragma unroll
  for (int j = 0; j < WideStage::kPerThread; ++j) {
    const int i = tid + WideStage::kThreads * j;
    const int g = i >> 10, r = i & 1023, ch = r >> 2, qe = r & 3;
    const int l = ch >> 2, c = ch & 3;
    buf[g * kSlice + (c * 4 + qe) * kRow + l] = st.v[j];
  }
}

template <typename TIn, bool VEC, bool VEC4>
__global__ __launch_bounds__(64 * kWideTG * kWideEG) void route_wide_kernel(
    const TIn* __restrict__ x, const float* __restrict__ Wr, int64_t T, int D, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ gate) {
  constexpr int R = kWideR, EC = kWideEC, TG = kWideTG, EG = kWideEG;
  constexpr int EMAX = kWidePasses * EG * 16;
  __shared__ float4 wbuf[2][EG * kSlice];
  __shared__ float s_logit[TG][R][EMAX];
  __shared__ int s_sel_e[TG][R][EMAX];
  __shared__ float s_sel_v[TG][R][EMAX];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int g = wave % EG, tg = wave / EG;
  const int64_t t0 = ((int64_t)blockIdx.x * TG + tg) * R;
  const int r = lane / EC, sub = lane % EC;

  const TIn* rows[R];
#pragma unroll
  for (int i = 0; i < R; ++i) rows[i] = x + (t0 + i < T ? t0 + i : T - 1) * D;
  // steps of 256 channels from a per-workgroup starting step (spreads the
  // workgroups' Wr reads over the L2 channels)
  constexpr int kStep = 64 * kCPL;
  const int nsteps = (D + kStep - 1) / kStep;
  const int s0 = (int)(blockIdx.x % (unsigned)nsteps);
  auto step_base = [&](int i) {
    const int st = s0 + i;
    return (st >= nsteps ? st - nsteps : st) * kStep;
  };
  const int npass = (E + EG * 16 - 1) / (EG * 16);
  for (int pass = 0; pass < npass; ++pass) {
    const int eb = pass * EG * 16;
    float acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.f;
    Raw4<TIn, VEC> xn[R];
    {
      const int d = step_base(0) + lane * kCPL;
#pragma unroll
      for (int i = 0; i < R; ++i) load4<TIn, VEC>(rows[i], d, D, d < D, xn[i]);
    }
    WideStage st;
    wide_stage_load<VEC4>(Wr, D, E, eb, step_base(0), tid, st);
    wide_stage_store(wbuf[0], tid, st);
    __syncthreads();
    int buf = 0;
    for (int i = 0; i < nsteps; ++i, buf ^= 1) {
      const int d = step_base(i) + lane * kCPL;
      const bool ok = d < D;
      const bool more = i + 1 < nsteps;
      float xv[R][kCPL];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (step_base(i) + kStep <= D)  // a whole step (uniform): no masking
          cvt4<TIn, VEC, false>(xn[j], d, D, ok, xv[j]);
        else
          cvt4<TIn, VEC, true>(xn[j], d, D, ok, xv[j]);
      }
      if (more) {
        // the stage first: waiting for it below leaves the x loads in flight
        const int dcn = step_base(i + 1), dn = dcn + lane * kCPL;
        wide_stage_load<VEC4>(Wr, D, E, eb, dcn, tid, st);
#pragma unroll
        for (int j = 0; j < R; ++j) load4<TIn, VEC>(rows[j], dn, D, dn < D, xn[j]);
      }
      const float4* wb = wbuf[buf] + g * kSlice;
#pragma unroll
      for (int c = 0; c < kCPL; ++c) {
        float w[EC];
#pragma unroll
        for (int qe = 0; qe < EC / 4; ++qe) {
          const float4 v = wb[(c * (EC / 4) + qe) * kRow + lane];
          w[4 * qe + 0] = v.x;
          w[4 * qe + 1] = v.y;
          w[4 * qe + 2] = v.z;
          w[4 * qe + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int e = 0; e < EC; ++e) acc[j * EC + e] = fmaf(xv[j][c], w[e], acc[j * EC + e]);
      }
      if (more) wide_stage_store(wbuf[buf ^ 1], tid, st);
      __syncthreads();
    }
    // transpose-reduce (as the 16-expert router): lane l ends with the logit
    // of (token l / 16, expert eb + 16 g + l % 16)
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
    s_logit[tg][r][eb + g * 16 + sub] = acc[0];
  }
  __syncthreads();
  if (g != 0) return;  // no barrier below

  // top k of token r among its E experts, (logit desc, expert asc): lane sub
  // holds experts sub, sub + 16, ...
  constexpr int NQ = EMAX / 16;
  const int64_t t = t0 + r;
  float val[NQ];
  bool taken[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    val[q] = s_logit[tg][r][q * 16 + sub];
    taken[q] = false;
  }
  float m0 = 0.f, z = 0.f;
  for (int j = 0; j < k; ++j) {
    // the lane's best untaken expert (ascending order keeps the lower index
    // on equal logits)
    bool cand = false;
    float bv = 0.f;
    int be = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 16 + sub;
      const bool c = e < E && !taken[q];
      if (c && (!cand || val[q] > bv)) {
        bv = val[q];
        be = e;
        cand = true;
      }
    }
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
    if (be % 16 == sub) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (q == be / 16) taken[q] = true;
    }
    if (j == 0) m0 = bv;
    if (sub == 0) {
      s_sel_e[tg][r][j] = be;
      s_sel_v[tg][r][j] = bv;
    }
    z += hw_exp2((bv - m0) * kLog2e);
  }
  // the token's 16 lanes write its k slots (the sums are wave-ordered: read
  // back after the wave's own LDS stores)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (t < T) {
    for (int j = sub; j < k; j += EC) {
      idx[t * k + j] = s_sel_e[tg][r][j];
      gate[t * k + j] = hw_exp2((s_sel_v[tg][r][j] - m0) * kLog2e) / z;
    }
  }
}

template <typename TIn>
int launch_route_wide_t(const void* x, const float* Wr, int64_t T, int D, int E, int k,
                        int32_t* idx, float* gate, hipStream_t s) {
  const int64_t per_wg = (int64_t)kWideTG * kWideR;
  const dim3 grid((unsigned)((T + per_wg - 1) / per_wg)), block(64 * kWideTG * kWideEG);
  const size_t vec_bytes = sizeof(TIn) * kCPL;
  const bool vec = ((size_t)D * sizeof(TIn)) % vec_bytes == 0 &&
                   reinterpret_cast<uintptr_t>(x) % vec_bytes == 0;
  const TIn* xp = static_cast<const TIn*>(x);
  const bool vec4 = E % 4 == 0 && reinterpret_cast<uintptr_t>(Wr) % 16 == 0;
  if (vec && vec4)
    hipLaunchKernelGGL((route_wide_kernel<TIn, true, true>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  else if (vec)
    hipLaunchKernelGGL((route_wide_kernel<TIn, true, false>), grid, block, 0, s, xp, Wr, T, D, E,
                       k, idx, gate);
  else
    hipLaunchKernelGGL((route_wide_kernel<TIn, false, false>), grid, block, 0, s, xp, Wr, T, D,
                       E, k, idx, gate);
  return hipGetLastError() == hipSuccess ? SWIMBA_OK : SWIMBA_EHIP;
}

}  // namespace router
}  // namespace swimba
