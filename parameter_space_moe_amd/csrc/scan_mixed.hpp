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
// (routing, gates, B_t, C_t) is wave-uniform: a per-wave LDS ring stages it one
// block of 8 tokens ahead, while x, dt_raw and y stream as coalesced 64-lane rows.  The expert tables
// A[e, tile, :], dt_bias and Dskip of the wave's 64 channels are staged once in
// LDS and read back as conflict-free 16-byte rows for the selected experts.
// The waves of a workgroup are consecutive chunks of the same channel tile and
// share that table.
//
// Long sequences are cut into chunks so that enough waves run at once.  Chunks
// are joined in three passes, all exact up to fp32 rounding:
//   1. chunk pass: every chunk from a zero state (chunk 0 from h0); it writes
//      provisional y, its end state, and its total decay
//      P[n] = prod_t exp(Delta_t Abar_t[n]) = exp2(sum_t m_t[n]), with m_t the
//      token's mixed exponent Delta_t Abar_t[n] log2 e, summed in registers;
//   2. carry pass: h_in(c+1) = P(c) * h_in(c) + h_end(c), sequential over chunks;
//   3. fix-up pass: chunk c >= 1 re-runs from h_in(c), tracking the carried part
//      g = (prod of decays) * h_in.  With A < 0 and gates >= 0 every decay is in
//      (0, 1], so once |g| is below 2^-24 of the state on every lane the rest of
//      the chunk equals the provisional y to fp32 resolution and the pass stops.
//      When the contraction does not hold (flagged by the chunk pass) or the
//      caller asks for it, the whole chunk is recomputed.
#pragma once
#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace mixed {

using stage::kTB;
using stage::Ring;
using stage::ring_bytes;
using stage::wave_sync;

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

// LDS: the workgroup's expert table (64 channels) and per-wave staging rings.
// With a scalar transition per (expert, channel) the A table is [E][64] floats.
struct Smem {
  float4* A;   // [E][4][64]  A[e, d0+lane, 4q..4q+3]  (scalar A: [E][64] floats)
  float2* BD;  // [E][64]     (dt_bias, Dskip)
  Ring ring;   // this wave's ring
};

__host__ __device__ inline size_t a_table_bytes(int E, bool scalar_a) {
  return scalar_a ? (size_t)E * 64 * 4 : (size_t)E * 4 * 64 * 16;
}

__device__ __forceinline__ Smem smem_layout(int E, int k, int wave, bool scalar_a) {
  extern __shared__ float4 smem_raw[];
  Smem s;
  char* p = reinterpret_cast<char*>(smem_raw);
  s.A = reinterpret_cast<float4*>(p);
  p += a_table_bytes(E, scalar_a);
  s.BD = reinterpret_cast<float2*>(p);
  p += (size_t)E * 64 * 8;
  p += ring_bytes(k) * wave;
  s.ring.bc = reinterpret_cast<float*>(p);
  s.ring.e = reinterpret_cast<int32_t*>(p + 2 * kTB * 32 * 4);
  s.ring.g = reinterpret_cast<float*>(p + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);
  return s;
}

__host__ inline size_t smem_bytes(int E, int k, int waves, bool scalar_a) {
  return a_table_bytes(E, scalar_a) + (size_t)E * 64 * 8 + ring_bytes(k) * waves;
}

// State update and readout of one token for one lane, given the per-state
// exponents m[n] = Delta Abar[n] log2(e) (SA: one exponent m[0]) and the
// Euler input dx = Delta x; B_t/C_t come from ring slot `slot`, position `i`.
template <bool TRACK, bool SA, bool ZOH>
__device__ __forceinline__ float update_readout(const Smem& s, int slot, int i, const float* m,
                                                float dx, float* h, float* g) {
  const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
  const float a0 = SA ? hw_exp2(m[0]) : 0.f;
  const float dx0 = (SA && ZOH) ? dx * zoh_phi(a0, m[0]) : dx;
  float yv = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 b4 = bc[q], c4 = bc[4 + q];
    const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * q + r;
      const float a = SA ? a0 : hw_exp2(m[n]);
      const float inj = (ZOH && !SA) ? (dx * bv[r]) * zoh_phi(a, m[n]) : dx0 * bv[r];
      h[n] = fmaf(a, h[n], inj);
      yv = fmaf(cv[r], h[n], yv);
      if (TRACK && !SA) g[n] *= a;
    }
  }
  if (TRACK && SA) g[0] *= a0;
  return yv;
}

// One token of the mixed recurrence for one lane with k == K known at compile
// time.  Routing (experts e[j], gates gw[j]) is wave-uniform.  All of the
// token's table reads (dt_bias/Dskip and the A rows) are issued together.
// ACC_U: add the token's exponents m[n] to the chunk's sums ms[n] (registers).
template <int K, bool TRACK, bool ACC_U, bool SA, bool ZOH>
__device__ __forceinline__ float mix_token_k(const Smem& s, float* ms, const int* e,
                                             const float* gw, int slot, int i, int lane,
                                             float xv, float rv, float* h, float* g) {
  float2 bd[K];
  float4 ar[SA ? 1 : K][4];
  float as[K];
  const float* Asc = reinterpret_cast<const float*>(s.A);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    bd[j] = s.BD[e[j] * 64 + lane];
    if constexpr (SA) {
      as[j] = Asc[e[j] * 64 + lane];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) ar[j][q] = s.A[(e[j] * 4 + q) * 64 + lane];
    }
  }
  // mixed dt_bias and Dskip
  float beta = 0.f, delta = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    beta = fmaf(gw[j], bd[j].x, beta);
    delta = fmaf(gw[j], bd[j].y, delta);
  }
  const float dlt = softplus_f32(rv + beta);
  const float dl2 = dlt * kLog2e;
  float u[K];
#pragma unroll
  for (int j = 0; j < K; ++j) u[j] = dl2 * gw[j];
  // mixed exponents m[n] = sum_j u_j A[e_j, d, n]
  float m[SA ? 1 : kN];
  if constexpr (SA) {
    m[0] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) m[0] = fmaf(u[j], as[j], m[0]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = ar[0][q];
      m[4 * q + 0] = u[0] * a.x;
      m[4 * q + 1] = u[0] * a.y;
      m[4 * q + 2] = u[0] * a.z;
      m[4 * q + 3] = u[0] * a.w;
    }
#pragma unroll
    for (int j = 1; j < K; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = ar[j][q];
        m[4 * q + 0] = fmaf(u[j], a.x, m[4 * q + 0]);
        m[4 * q + 1] = fmaf(u[j], a.y, m[4 * q + 1]);
        m[4 * q + 2] = fmaf(u[j], a.z, m[4 * q + 2]);
        m[4 * q + 3] = fmaf(u[j], a.w, m[4 * q + 3]);
      }
  }
  if (ACC_U)
#pragma unroll
    for (int n = 0; n < (SA ? 1 : kN); ++n) ms[n] += m[n];
  const float yv = update_readout<TRACK, SA, ZOH>(s, slot, i, m, dlt * xv, h, g);
  return fmaf(delta, xv, yv);
}

// One token of the mixed recurrence for one lane.  Routing (experts e[j],
// gates g[j], j < k) is wave-uniform; B_t/C_t come from ring slot `slot`,
// position `i`.  Every LDS address below depends only on (e, lane), so all of
// a token's reads can be in flight together.
//   K > 0: k == K known at compile time (mix_token_k); K == 0: runtime k.
//   TRACK: also decay the carried part g (fix-up pass; with SA, g[0] is the
//          carried part's common decay factor).
//   ACC_U: add the token's exponents to the chunk's sums ms (chunk pass).
//   SA: one transition per (expert, channel), shared by the 16 states (the
//       Mamba-2 form A = a I): one exponential per token instead of 16.
//   ZOH: zero-order-hold input term, zoh_phi(a) times the Euler term.
template <int K, bool TRACK, bool ACC_U, bool SA, bool ZOH>
__device__ __forceinline__ float mix_token(const MixParams& p, const Smem& s, float* ms,
                                           const int* e, const float* gw, int slot, int i,
                                           int lane, float xv, float rv, float* h, float* g) {
  if constexpr (K > 0)
    return mix_token_k<K, TRACK, ACC_U, SA, ZOH>(s, ms, e, gw, slot, i, lane, xv, rv, h, g);
  const int k = K > 0 ? K : p.k;
  // mixed dt_bias and Dskip
  float beta = 0.f, delta = 0.f;
  auto bias_slot = [&](int j) {
    const float2 bd = s.BD[e[j] * 64 + lane];
    beta = fmaf(gw[j], bd.x, beta);
    delta = fmaf(gw[j], bd.y, delta);
  };
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) bias_slot(j);
  } else {
    for (int j = 0; j < k; ++j) bias_slot(j);
  }
  const float dlt = softplus_f32(rv + beta);
  if constexpr (SA) {
    // mixed exponent Delta * sum_j g_j A[e_j, d] * log2(e), one per token
    const float dl2 = dlt * kLog2e;
    const float* As = reinterpret_cast<const float*>(s.A);
    float m = 0.f;
    auto a_slot = [&](int j) {
      const float u = dl2 * gw[j];
      m = fmaf(u, As[e[j] * 64 + lane], m);
    };
    if constexpr (K > 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) a_slot(j);
    } else {
      for (int j = 0; j < k; ++j) a_slot(j);
    }
    if (ACC_U) ms[0] += m;
    const float a = hw_exp2(m);
    const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
    const float dx = ZOH ? dlt * xv * zoh_phi(a, m) : dlt * xv;
    float yv = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 b4 = bc[q], c4 = bc[4 + q];
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 4 * q + r;
        h[n] = fmaf(a, h[n], dx * bv[r]);
        yv = fmaf(cv[r], h[n], yv);
      }
    }
    if (TRACK) g[0] *= a;
    return fmaf(delta, xv, yv);
  }
  // mixed exponent m[n] = Delta * sum_j g_j A[e_j, d, n] * log2(e)
  float m[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) m[n] = 0.f;
  const float dl2 = dlt * kLog2e;
  auto a_slot = [&](int j) {
    const float u = dl2 * gw[j];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = s.A[(e[j] * 4 + q) * 64 + lane];
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
  if (ACC_U)
#pragma unroll
    for (int n = 0; n < kN; ++n) ms[n] += m[n];
  const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
  const float dx = dlt * xv;
  float yv = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 b4 = bc[q], c4 = bc[4 + q];
    const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * q + r;
      const float a = hw_exp2(m[n]);
      const float inj = ZOH ? (dx * bv[r]) * zoh_phi(a, m[n]) : dx * bv[r];
      h[n] = fmaf(a, h[n], inj);
      yv = fmaf(cv[r], h[n], yv);
      if (TRACK) g[n] *= a;
    }
  }
  return fmaf(delta, xv, yv);
}

// Walk tokens [t0, t1) of sequence b for one lane, staging each block of kTB
// tokens' uniform data and x/dt_raw one block ahead.  With TRACK and
// `truncate`, stops once the carried part g has decayed on every lane.
// x, dt_raw and y go through per-block buffer resources (scalar token offsets,
// a fixed per-lane channel offset); the prefetch of the next block is issued
// before the current one computes and is waited on only when it is used.
template <typename TIn, typename TOut, int K, bool TRACK, bool ACC_U, bool SA, bool ZOH>
__device__ __forceinline__ void walk(const MixParams& p, const Smem& s, float* ms, int b, int t0,
                                     int t1, int d, bool active, bool full_tile, int lane,
                                     bool truncate, float* h, float* g, int& gate_bad) {
  constexpr int KW = (kTB * (K > 0 ? K : 16) + 63) / 64;
  const int k = K > 0 ? K : p.k;
  const int D = p.D;
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  // lanes past D (ragged tile) read 0 and store nothing
  const uint32_t xoff = active ? (uint32_t)d * (uint32_t)sizeof(TIn) : stage::kOffNone;
  const uint32_t yoff = (uint32_t)d * (uint32_t)sizeof(TOut);
  const uint32_t xrow = (uint32_t)D * (uint32_t)sizeof(TIn);
  const uint32_t yrow = (uint32_t)D * (uint32_t)sizeof(TOut);
  TIn xc[kTB], rc[kTB], xn[kTB], rn[kTB];
  stage::Stager<TIn, KW> st;
  st.init(lane);
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  auto load_xr = [&](int t, TIn* xs, TIn* rs) {
    const int v = valid_at(t);
    const stage::rsrc_t rx = stage::rows_rsrc<TIn>(p.x, row + t, v, D);
    const stage::rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, row + t, v, D);
    // the scalar offset is not range-checked by the hardware: rows past the
    // tensor's end re-read its last row
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const uint32_t so = (uint32_t)min(i, v - 1) * xrow;
      xs[i] = stage::buf_load<TIn>(rx, xoff, so);
      rs[i] = stage::buf_load<TIn>(rr, xoff, so);
    }
  };

  st.issue(p, row + t0, valid_at(t0), k);
  load_xr(t0, xc, rc);
  st.commit(s.ring, 0, min(kTB, t1 - t0), k, p.E, lane, gate_bad);

  int slot = 0;
  for (int tb = t0; tb < t1; tb += kTB, slot ^= 1) {
    const int n = min(kTB, t1 - tb);
    const int tn = tb + kTB;
    const bool more = tn < t1;
    if (more) {
      st.issue(p, row + tn, valid_at(tn), k);
      load_xr(tn, xn, rn);
    }
    wave_sync();
    // stores past the block's n tokens fall outside this buffer and are dropped
    const stage::rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, n, D);
    // full blocks on full tiles run as one branch-free basic block of kTB
    // tokens, so the scheduler can overlap a token's LDS reads with the
    // previous token's arithmetic; the ragged tail keeps its guards
    const bool fast = n == kTB && full_tile;
    if constexpr (K > 0) {
      if (fast) {
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          int ev[K];
          float gv[K];
#pragma unroll
          for (int j = 0; j < K; ++j) {
            ev[j] = s.ring.e[(slot * kTB + i) * K + j];
            gv[j] = s.ring.g[(slot * kTB + i) * K + j];
          }
          const float yv = mix_token<K, TRACK, ACC_U, SA, ZOH>(p, s, ms, ev, gv, slot, i, lane,
                                                      to_f32(xc[i]), to_f32(rc[i]), h, g);
          stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      } else {
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
          if (i < n) {
            int ev[K];
            float gv[K];
#pragma unroll
            for (int j = 0; j < K; ++j) {
              ev[j] = s.ring.e[(slot * kTB + i) * K + j];
              gv[j] = s.ring.g[(slot * kTB + i) * K + j];
            }
            const float xv = active ? to_f32(xc[i]) : 0.f, rv = active ? to_f32(rc[i]) : 0.f;
            const float yv = mix_token<K, TRACK, ACC_U, SA, ZOH>(p, s, ms, ev, gv, slot, i, lane, xv, rv,
                                                        h, g);
            if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          int eb[16];
          float gb[16];
          for (int j = 0; j < k; ++j) {
            eb[j] = s.ring.e[(slot * kTB + i) * k + j];
            gb[j] = s.ring.g[(slot * kTB + i) * k + j];
          }
          const float xv = active ? to_f32(xc[i]) : 0.f, rv = active ? to_f32(rc[i]) : 0.f;
          const float yv = mix_token<K, TRACK, ACC_U, SA, ZOH>(p, s, ms, eb, gb, slot, i, lane, xv, rv, h,
                                                      g);
          if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      }
    }
    if (TRACK && truncate) {
      float mh = 0.f;
#pragma unroll
      for (int q = 0; q < kN; ++q) mh = fmaxf(mh, fabsf(h[q]));
      const float thr = fmaxf(kFixupTol * mh, kTiny);
      bool conv = true;
      if constexpr (SA) {
        conv = fabsf(g[0]) * g[1] <= thr;  // g[1] = max_n |h_in[n]|; NaN: not converged
      } else {
#pragma unroll
        for (int q = 0; q < kN; ++q) conv &= fabsf(g[q]) <= thr;  // NaN: not converged
      }
      if (__all(conv)) break;
    }
    if (more) {
      st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        xc[i] = xn[i];
        rc[i] = rn[i];
      }
    }
  }
}

// Pass 1 (or the only pass when CHUNKED is false).
template <typename TIn, typename TOut, int WAVES, int K, bool CHUNKED, bool SA, bool ZOH>
__global__ __launch_bounds__(WAVES * 64) void mix_chunk_kernel(MixParams p) {
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const Smem s = smem_layout(p.E, K > 0 ? K : p.k, wave, SA);
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  int bad = stage::load_table(p, s.A, s.BD, d0, SA);
  bad = __syncthreads_or(bad);

  const int c = cg * WAVES + wave;
  if (c >= p.nchunks) return;  // no barrier below
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n)
    h[n] = (c == 0 && p.h0 != nullptr && active) ? p.h0[((size_t)b * p.D + d) * kN + n] : 0.f;

  // every chunk writes y (provisional for chunks >= 1, recomputed by the
  // fix-up pass where the carried-in state still matters)
  int gate_bad = 0;
  // the chunk's summed exponents (SA: ms[0] only)
  float ms[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) ms[n] = 0.f;
  walk<TIn, TOut, K, false, CHUNKED, SA, ZOH>(p, s, ms, b, t0, t1, d, active, d0 + 64 <= p.D,
                                              lane, false, h, nullptr, gate_bad);

  if (CHUNKED) {
    // total decay of the chunk: P[n] = exp2(sum_t m_t[n]); with SA one decay
    // per channel, written to every state row for the carry pass
    if (active) {
      const size_t base = (((size_t)b * p.nchunks + c) * kN) * p.D + d;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        p.P[base + (size_t)n * p.D] = hw_exp2(ms[SA ? 0 : n]);
        p.H[base + (size_t)n * p.D] = h[n];
      }
    }
    gate_bad = __any(gate_bad);
    if (lane == 0) p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] = (bad | gate_bad) ? 1 : 0;
  } else if (p.h_final != nullptr && active) {
#pragma unroll
    for (int n = 0; n < kN; ++n) p.h_final[((size_t)b * p.D + d) * kN + n] = h[n];
  }
}

// Pass 3: chunks 1.. re-run from their carried-in state until the carried part
// has decayed away (or to the chunk's end).
template <typename TIn, typename TOut, int WAVES, int K, bool SA, bool ZOH>
__global__ __launch_bounds__(WAVES * 64) void mix_fixup_kernel(MixParams p) {
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const Smem s = smem_layout(p.E, K > 0 ? K : p.k, wave, SA);
  const int nfix = p.nchunks - 1;
  const int ncg = (nfix + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  stage::load_table(p, s.A, s.BD, d0, SA);
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
  if (SA) {
    // the carried part is G * h_in: track G and max |h_in|
    float mh = 0.f;
#pragma unroll
    for (int n = 0; n < kN; ++n) mh = fmaxf(mh, fabsf(h[n]));
    g[0] = 1.f;
    g[1] = mh;
  }
  const bool truncate = p.carry == SWIMBA_CARRY_FIXUP &&
                        p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] == 0;
  int gate_bad = 0;
  walk<TIn, TOut, K, true, false, SA, ZOH>(p, s, nullptr, b, t0, t1, d, active, d0 + 64 <= p.D, lane,
                                  truncate, h, g, gate_bad);
}

template <typename TIn, typename TOut, int WAVES, int K, bool SA, bool ZOH>
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

  const size_t smem1 = smem_bytes(p.E, p.k, WAVES, SA);
  const size_t smem3 = smem1;
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  if (pl.nchunks <= 1) {
    p.nchunks = 1;
    dim3 grid((unsigned)((size_t)p.B * p.ntiles));
    allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH>, smem3);
    const int rc = launch_timed(mix_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH>, grid,
                                dim3(WAVES * 64), smem3, st, ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  dim3 grid1((unsigned)((size_t)p.B * ncg * p.ntiles));
  allow_dynamic_lds(mix_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH>, smem1);
  int rc = launch_timed(mix_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH>, grid1, dim3(WAVES * 64),
                        smem1, st, ev, p);
  if (rc != SWIMBA_OK) return rc;
  rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 0, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  const int ncg3 = (p.nchunks - 1 + WAVES - 1) / WAVES;
  dim3 grid3((unsigned)((size_t)p.B * ncg3 * p.ntiles));
  allow_dynamic_lds(mix_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH>, smem3);
  return launch_timed(mix_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH>, grid3, dim3(WAVES * 64), smem3, st,
                      ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut, int WAVES, bool SA, bool ZOH>
int launch_mixed_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_mixed_t<TIn, TOut, WAVES, 1, SA, ZOH>(a, pl, ws, st);
    case 2:
      return launch_mixed_t<TIn, TOut, WAVES, 2, SA, ZOH>(a, pl, ws, st);
    default:
      return launch_mixed_t<TIn, TOut, WAVES, 0, SA, ZOH>(a, pl, ws, st);
  }
}

template <typename TIn, typename TOut, int WAVES, bool SA>
int launch_mixed_z(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->disc == SWIMBA_DISC_ZOH) return launch_mixed_k<TIn, TOut, WAVES, SA, true>(a, pl, ws, st);
  return launch_mixed_k<TIn, TOut, WAVES, SA, false>(a, pl, ws, st);
}

template <typename TIn, typename TOut>
int launch_mixed_w(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->a_form == SWIMBA_A_SCALAR) {
    if (pl.waves == 8) return launch_mixed_z<TIn, TOut, 8, true>(a, pl, ws, st);
    return launch_mixed_z<TIn, TOut, 4, true>(a, pl, ws, st);
  }
  if (pl.waves == 8) return launch_mixed_z<TIn, TOut, 8, false>(a, pl, ws, st);
  return launch_mixed_z<TIn, TOut, 4, false>(a, pl, ws, st);
}

}  // namespace mixed
}  // namespace swimba
