// Parameter-space-mixed selective scan (Swimba) for gfx950.
//
// Pages: "Swimba: Switch Mamba Model Scales State Space Models" (Dutch summary,
// "Kernmechanisme van Swimba": the selected experts' parameters are mixed with
// the router weights and one recurrence runs; Theorem 1: the result is a single
// selective SSM; Theorem 3: contractive transitions keep it stable) and
// "Mamba y las SSMs: el retorno del estado persistente" ("Mamba": transition
// exp(Delta A), selective B_t and C_t; Figure 2: the state stays on chip while
// inputs and outputs stream from HBM).
//
// Layout of the work.  A lane owns one channel d of one sequence b and keeps its
// 16 fp32 states in VGPRs for a whole chunk of tokens.  The 64 lanes of a wave
// are 64 consecutive channels of the same token, so everything per token
// (routing, gates, B_t, C_t) is wave-uniform and read through the scalar unit,
// while x, dt_raw and y stream as coalesced 64-lane rows.  The expert tables
// A[e, tile, :], dt_bias and Dskip of the wave's 64 channels are staged once in
// LDS and read back as conflict-free 16-byte rows for the selected experts.
// The waves of a workgroup are consecutive chunks of the same channel tile and
// share that table.
//
// Long sequences are cut into chunks so that enough waves run at once.  Chunks
// are joined in three passes, all exact up to fp32 rounding:
//   1. chunk pass: every chunk from a zero state (chunk 0 from h0); it writes
//      provisional y, its end state, and its total decay
//      P[n] = prod_t exp(Delta_t Abar_t[n]) = exp2(sum_e U_e A[e,n] log2 e),
//      with U_e the gate-weighted Delta of expert e summed over the chunk;
//   2. carry pass: h_in(c+1) = P(c) * h_in(c) + h_end(c), sequential over chunks;
//   3. fix-up pass: chunk c >= 1 re-runs from h_in(c), tracking the carried part
//      g = (prod of decays) * h_in.  With A < 0 and gates >= 0 every decay is in
//      (0, 1], so once |g| is below 2^-24 of the state on every lane the rest of
//      the chunk equals the provisional y to fp32 resolution and the pass stops.
//      When the contraction does not hold (flagged by the chunk pass) or the
//      caller asks for it, the whole chunk is recomputed.
#pragma once
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace mixed {

constexpr float kFixupTol = 5.9604645e-08f;  // 2^-24
constexpr float kTiny = 1e-30f;

struct MixParams {
  int B, L, D, E, k;
  int chunk, nchunks, ntiles;
  int carry;  // SWIMBA_CARRY_REWALK or SWIMBA_CARRY_FIXUP
  const void* x;
  const void* dt;
  const void* Bm;
  const void* Cm;
  const int32_t* idx;
  const float* gate;
  const float* A;
  const float* bias;
  const float* Dsk;
  const float* h0;
  void* y;
  float* h_final;
  float* P;           // [B][C][16][D] chunk decays
  float* H;           // [B][C][16][D] chunk end states, then carried-in states
  int32_t* flags;     // [B][C][ntiles] 1 = contraction not guaranteed
};

// LDS: table of the workgroup's 64 channels plus per-wave decay accumulators.
struct Smem {
  float4* A;   // [E][4][64]  A[e, d0+lane, 4q..4q+3]
  float2* BD;  // [E][64]     (dt_bias, Dskip)
  float* U;    // [waves][E][64]
};

__device__ __forceinline__ Smem smem_layout(int E, bool with_table) {
  extern __shared__ float4 smem_raw[];
  Smem s;
  float4* p = smem_raw;
  if (with_table) {
    s.A = p;
    p += E * 4 * 64;
    s.BD = reinterpret_cast<float2*>(p);
    p += E * 64 / 2;
  } else {
    s.A = nullptr;
    s.BD = nullptr;
  }
  s.U = reinterpret_cast<float*>(p);
  return s;
}

// Stage the tile's expert parameters; returns 1 if any A in the tile is not
// strictly negative (including NaN).
__device__ __forceinline__ int load_table(const MixParams& p, const Smem& s, int d0) {
  int bad = 0;
  const int nthr = blockDim.x;
  for (int i = threadIdx.x; i < p.E * 256; i += nthr) {
    int e = i >> 8, r = i & 255, dl = r >> 2, q = r & 3;
    int d = d0 + dl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d < p.D) {
      const float* a = p.A + ((size_t)e * p.D + d) * kN + q * 4;
      v = make_float4(a[0], a[1], a[2], a[3]);
      bad |= !(v.x < 0.f) | !(v.y < 0.f) | !(v.z < 0.f) | !(v.w < 0.f);
    }
    s.A[(e * 4 + q) * 64 + dl] = v;
  }
  for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
    int e = i >> 6, dl = i & 63, d = d0 + dl;
    float2 v = make_float2(0.f, 0.f);
    if (d < p.D) v = make_float2(p.bias[(size_t)e * p.D + d], p.Dsk[(size_t)e * p.D + d]);
    s.BD[i] = v;
  }
  return bad;
}

// Routing slot j of token bt (wave-uniform), clamped into range.
__device__ __forceinline__ int slot_expert(const MixParams& p, size_t bt, int j) {
  int e = p.idx[bt * p.k + j];
  e = e < 0 ? 0 : e;
  return e >= p.E ? p.E - 1 : e;
}

// One token of the mixed recurrence for one lane.
//   K > 0: k == K known at compile time; K == 0: runtime k.
//   TRACK: also decay the carried part g (fix-up pass).
//   ACC_U: accumulate gate-weighted Delta per expert (chunk pass).
template <int K, typename TIn, bool TRACK, bool ACC_U>
__device__ __forceinline__ float mix_token(const MixParams& p, const Smem& s, float* U,
                                           size_t bt, int lane, float xv, float rv, float* h,
                                           float* g, int& gate_bad) {
  const int k = K > 0 ? K : p.k;
  // mixed dt_bias and Dskip
  float beta = 0.f, delta = 0.f;
  auto bias_slot = [&](int j) {
    const int e = slot_expert(p, bt, j);
    const float gj = p.gate[bt * k + j];
    gate_bad |= !(gj >= 0.f);
    const float2 bd = s.BD[e * 64 + lane];
    beta = fmaf(gj, bd.x, beta);
    delta = fmaf(gj, bd.y, delta);
  };
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) bias_slot(j);
  } else {
    for (int j = 0; j < k; ++j) bias_slot(j);
  }
  const float dlt = softplus_f32(rv + beta);
  // mixed exponent m[n] = Delta * sum_j g_j A[e_j, d, n] * log2(e)
  float m[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) m[n] = 0.f;
  const float dl2 = dlt * kLog2e;
  auto a_slot = [&](int j) {
    const int e = slot_expert(p, bt, j);
    const float u = dl2 * p.gate[bt * k + j];
    if (ACC_U) atomicAdd(&U[e * 64 + lane], u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = s.A[(e * 4 + q) * 64 + lane];
      if (K > 0 && j == 0) {
        m[4 * q + 0] = u * a.x;
        m[4 * q + 1] = u * a.y;
        m[4 * q + 2] = u * a.z;
        m[4 * q + 3] = u * a.w;
      } else {
        m[4 * q + 0] = fmaf(u, a.x, m[4 * q + 0]);
        m[4 * q + 1] = fmaf(u, a.y, m[4 * q + 1]);
        m[4 * q + 2] = fmaf(u, a.z, m[4 * q + 2]);
        m[4 * q + 3] = fmaf(u, a.w, m[4 * q + 3]);
      }
    }
  };
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) a_slot(j);
  } else {
    for (int j = 0; j < k; ++j) a_slot(j);
  }
  const TIn* Bp = reinterpret_cast<const TIn*>(p.Bm) + bt * kN;
  const TIn* Cp = reinterpret_cast<const TIn*>(p.Cm) + bt * kN;
  const float dx = dlt * xv;
  float yv = 0.f;
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    float a = hw_exp2(m[n]);
    h[n] = fmaf(a, h[n], dx * to_f32(Bp[n]));
    yv = fmaf(to_f32(Cp[n]), h[n], yv);
    if (TRACK) g[n] *= a;
  }
  return fmaf(delta, xv, yv);
}

// Pass 1 (or the only pass when CHUNKED is false).
template <typename TIn, typename TOut, int WAVES, int K, bool CHUNKED>
__global__ __launch_bounds__(WAVES * 64) void mix_chunk_kernel(MixParams p) {
  const Smem s = smem_layout(p.E, true);
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  int bad = load_table(p, s, d0);
  float* U = s.U + wave * p.E * 64;
  if (CHUNKED)
    for (int e = 0; e < p.E; ++e) U[e * 64 + lane] = 0.f;
  bad = __syncthreads_or(bad);

  const int c = cg * WAVES + wave;
  if (c >= p.nchunks) return;  // no barrier below
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n)
    h[n] = (c == 0 && p.h0 != nullptr && active) ? p.h0[((size_t)b * p.D + d) * kN + n] : 0.f;

  const bool write_y = !CHUNKED || c == 0 || p.carry != SWIMBA_CARRY_REWALK;
  const TIn* X = reinterpret_cast<const TIn*>(p.x);
  const TIn* R = reinterpret_cast<const TIn*>(p.dt);
  TOut* Y = reinterpret_cast<TOut*>(p.y);
  int gate_bad = 0;
  const int dd = active ? d : 0;
  size_t bt = (size_t)b * p.L + t0;
  size_t off = bt * p.D + dd;
  // software pipeline: the next token's x and dt_raw are in flight during the current one
  float xn = to_f32(X[off]), rn = to_f32(R[off]);
  for (int t = t0; t < t1; ++t, ++bt, off += p.D) {
    const float xv = active ? xn : 0.f, rv = active ? rn : 0.f;
    if (t + 1 < t1) {
      xn = to_f32(X[off + p.D]);
      rn = to_f32(R[off + p.D]);
    }
    float yv = mix_token<K, TIn, false, CHUNKED>(p, s, U, bt, lane, xv, rv, h, nullptr, gate_bad);
    if (write_y && active) Y[off] = from_f32<TOut>(yv);
  }

  if (CHUNKED) {
    // total decay of the chunk: P[n] = exp2(sum_e U_e A[e, d, n])
    float m[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) m[n] = 0.f;
    for (int e = 0; e < p.E; ++e) {
      float u = U[e * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 a = s.A[(e * 4 + q) * 64 + lane];
        m[4 * q + 0] = fmaf(u, a.x, m[4 * q + 0]);
        m[4 * q + 1] = fmaf(u, a.y, m[4 * q + 1]);
        m[4 * q + 2] = fmaf(u, a.z, m[4 * q + 2]);
        m[4 * q + 3] = fmaf(u, a.w, m[4 * q + 3]);
      }
    }
    if (active) {
      const size_t base = (((size_t)b * p.nchunks + c) * kN) * p.D + d;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        p.P[base + (size_t)n * p.D] = hw_exp2(m[n]);
        p.H[base + (size_t)n * p.D] = h[n];
      }
    }
    if (lane == 0) p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] = (bad | gate_bad) ? 1 : 0;
  } else if (p.h_final != nullptr && active) {
#pragma unroll
    for (int n = 0; n < kN; ++n) p.h_final[((size_t)b * p.D + d) * kN + n] = h[n];
  }
}

// Pass 3: chunks 1.. re-run from their carried-in state until the carried part
// has decayed away (or to the chunk's end).
template <typename TIn, typename TOut, int WAVES, int K>
__global__ __launch_bounds__(WAVES * 64) void mix_fixup_kernel(MixParams p) {
  const Smem s = smem_layout(p.E, true);
  const int nfix = p.nchunks - 1;
  const int ncg = (nfix + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  load_table(p, s, d0);
  __syncthreads();

  const int c = 1 + cg * WAVES + wave;
  if (c >= p.nchunks) return;
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);
  const size_t base = (((size_t)b * p.nchunks + c) * kN) * p.D + (active ? d : 0);
  float h[kN], g[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    h[n] = active ? p.H[base + (size_t)n * p.D] : 0.f;
    g[n] = h[n];
  }
  const bool truncate = p.carry == SWIMBA_CARRY_FIXUP &&
                        p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] == 0;
  const TIn* X = reinterpret_cast<const TIn*>(p.x);
  const TIn* R = reinterpret_cast<const TIn*>(p.dt);
  TOut* Y = reinterpret_cast<TOut*>(p.y);
  int gate_bad = 0;
  const int dd = active ? d : 0;
  size_t bt = (size_t)b * p.L + t0;
  size_t off = bt * p.D + dd;
  float xn = to_f32(X[off]), rn = to_f32(R[off]);
  for (int t = t0; t < t1; ++t, ++bt, off += p.D) {
    const float xv = active ? xn : 0.f, rv = active ? rn : 0.f;
    if (t + 1 < t1) {
      xn = to_f32(X[off + p.D]);
      rn = to_f32(R[off + p.D]);
    }
    float yv = mix_token<K, TIn, true, false>(p, s, nullptr, bt, lane, xv, rv, h, g, gate_bad);
    if (active) Y[off] = from_f32<TOut>(yv);
    if (truncate && ((t - t0) & 1)) {
      float mh = 0.f;
#pragma unroll
      for (int n = 0; n < kN; ++n) mh = fmaxf(mh, fabsf(h[n]));
      const float thr = fmaxf(kFixupTol * mh, kTiny);
      bool conv = true;
#pragma unroll
      for (int n = 0; n < kN; ++n) conv &= fabsf(g[n]) <= thr;  // NaN: not converged
      if (__all(conv)) break;
    }
  }
}

template <typename TIn, typename TOut, int WAVES, int K>
int launch_mixed_t(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  MixParams p;
  p.B = a->B;
  p.L = a->L;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.ntiles = pl.ntiles;
  p.carry = a->carry == SWIMBA_CARRY_REWALK ? SWIMBA_CARRY_REWALK : SWIMBA_CARRY_FIXUP;
  p.x = a->x;
  p.dt = a->dt_raw;
  p.Bm = a->Bm;
  p.Cm = a->Cm;
  p.idx = a->idx;
  p.gate = a->gate;
  p.A = a->A;
  p.bias = a->dt_bias;
  p.Dsk = a->Dskip;
  p.h0 = a->h0;
  p.y = a->y;
  p.h_final = a->h_final;
  char* w = static_cast<char*>(ws);
  p.P = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_P) : nullptr;
  p.H = pl.nchunks > 1 ? reinterpret_cast<float*>(w + pl.off_H) : nullptr;
  p.flags = pl.nchunks > 1 ? reinterpret_cast<int32_t*>(w + pl.off_flags) : nullptr;

  const size_t table = (size_t)p.E * (4 * 64 * 16 + 64 * 8);
  const size_t ubytes = (size_t)WAVES * p.E * 64 * 4;
  hipEvent_t* ev = a->phase_events;
  if (ev) (void)hipEventRecord(ev[0], st);
  if (pl.nchunks <= 1) {
    p.nchunks = 1;
    dim3 grid((unsigned)((size_t)p.B * p.ntiles));
    allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, false>, table);
    hipLaunchKernelGGL((mix_chunk_kernel<TIn, TOut, WAVES, K, false>), grid, dim3(WAVES * 64),
                       table, st, p);
    if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
    if (ev) {
      (void)hipEventRecord(ev[1], st);
      (void)hipEventRecord(ev[2], st);
      (void)hipEventRecord(ev[3], st);
    }
    return SWIMBA_OK;
  }
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  dim3 grid1((unsigned)((size_t)p.B * ncg * p.ntiles));
  allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, true>, table + ubytes);
  hipLaunchKernelGGL((mix_chunk_kernel<TIn, TOut, WAVES, K, true>), grid1, dim3(WAVES * 64),
                     table + ubytes, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  if (ev) (void)hipEventRecord(ev[1], st);
  const int rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 0, st);
  if (rc != SWIMBA_OK) return rc;
  if (ev) (void)hipEventRecord(ev[2], st);
  const int ncg3 = (p.nchunks - 1 + WAVES - 1) / WAVES;
  dim3 grid3((unsigned)((size_t)p.B * ncg3 * p.ntiles));
  allow_dynamic_lds(mix_fixup_kernel<TIn, TOut, WAVES, K>, table);
  hipLaunchKernelGGL((mix_fixup_kernel<TIn, TOut, WAVES, K>), grid3, dim3(WAVES * 64), table, st,
                     p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  if (ev) (void)hipEventRecord(ev[3], st);
  return SWIMBA_OK;
}

template <typename TIn, typename TOut, int WAVES>
int launch_mixed_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_mixed_t<TIn, TOut, WAVES, 1>(a, pl, ws, st);
    case 2:
      return launch_mixed_t<TIn, TOut, WAVES, 2>(a, pl, ws, st);
    default:
      return launch_mixed_t<TIn, TOut, WAVES, 0>(a, pl, ws, st);
  }
}

template <typename TIn, typename TOut>
int launch_mixed_w(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (pl.waves == 8) return launch_mixed_k<TIn, TOut, 8>(a, pl, ws, st);
  return launch_mixed_k<TIn, TOut, 4>(a, pl, ws, st);
}

}  // namespace mixed
}  // namespace swimba
