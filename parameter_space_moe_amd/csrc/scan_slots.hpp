// Separate trajectories per routing slot for gfx950: slot j of every (sequence,
// channel) keeps its own 16 states, which advance at every token with the
// parameters of the expert that the router put in slot j (its own A, dt_bias
// and Dskip, not mixed), and keep their value when that expert changes; the
// token's output adds the slots' outputs C_t . h_j + Dskip x weighted by the
// gates.  This is the other reading of separate trajectories next to one state
// per expert (pages: "Swimba: Switch Mamba Model Scales State Space Models",
// Spanish "Distinción de Diseños", French "Distinction des deux designs").
//
// Layout of the work, as in the mixed scan: a lane owns one channel and keeps
// all k x 16 slot states in VGPRs for a chunk of tokens; routing, gates, B_t
// and C_t are wave-uniform and staged per wave one block of 8 tokens ahead;
// x, dt_raw and y stream as coalesced 64-lane rows.  The expert tables of the
// tile (A rows, dt_bias, Dskip) sit in LDS and every slot reads its expert's
// row each token.  The gates never enter a state, so the transitions are
// contractive whenever A < 0, whatever the gates.
//
// More than 16 experts (MEM, k <= 2): no table; each slot reads its expert's
// A row, dt_bias and Dskip from memory (L2) every token, the chunk decays are
// summed per slot in registers, and a pre-pass checks every tile's A.
//
// Chunks are joined in the mixed scan's three passes, per slot: the chunk
// pass runs every chunk from zero and records each slot's end state and total
// decay P_j[n] = exp2(sum_e U_je A[e,n] log2 e) (U_je: Delta summed over the
// chunk's tokens whose slot j chose e); the carry pass joins the chunks; the
// fix-up pass re-runs chunks 1.. from their carried-in states until the
// carried part of every slot has decayed below fp32 resolution.
#pragma once
#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace slots {

using stage::kTB;
using stage::Ring;
using stage::ring_bytes;
using stage::wave_sync;

constexpr float kFixupTol = 5.9604645e-08f;  // 2^-24
constexpr float kTiny = 1e-30f;

struct SlotParams {
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
  const float* h0;    // [B][k][D][16]
  void* y;
  float* h_final;     // [B][k][D][16]
  float* P;           // [B][C][k*16][D] chunk decays
  float* H;           // [B][C][k*16][D] chunk end states, then carried-in states
  int32_t* flags;     // [B][C][ntiles] 1 = some A of the tile is not negative
  const int32_t* tflags;  // [ntiles] the same per tile (MEM: from the pre-pass)
};

// LDS: the tile's expert table, per-wave decay sums per (slot, expert) and
// per-wave staging rings.
struct Smem {
  float4* A;   // [E][4][64]  (scalar A: [E][64] floats)
  float2* BD;  // [E][64]     (dt_bias, Dskip)
  float* U;    // [waves][k][E][64] (chunk pass only)
  Ring ring;
};

__host__ __device__ inline size_t a_table_bytes(int E, bool scalar_a) {
  return scalar_a ? (size_t)E * 64 * 4 : (size_t)E * 4 * 64 * 16;
}

__host__ __device__ inline size_t u_bytes(int E, int k, int waves) {
  return (size_t)waves * k * E * 64 * 4;
}

__device__ __forceinline__ Smem smem_layout(int E, int k, bool with_u, int waves, int wave,
                                            bool scalar_a) {
  extern __shared__ float4 smem_raw[];
  Smem s;
  char* p = reinterpret_cast<char*>(smem_raw);
  s.A = reinterpret_cast<float4*>(p);
  p += a_table_bytes(E, scalar_a);
  s.BD = reinterpret_cast<float2*>(p);
  p += (size_t)E * 64 * 8;
  s.U = reinterpret_cast<float*>(p);
  if (with_u) p += u_bytes(E, k, waves);
  p += ring_bytes(k) * wave;
  s.ring.bc = reinterpret_cast<float*>(p);
  s.ring.e = reinterpret_cast<int32_t*>(p + 2 * kTB * 32 * 4);
  s.ring.g = reinterpret_cast<float*>(p + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);
  return s;
}

__host__ inline size_t smem_bytes(int E, int k, bool with_u, int waves, bool scalar_a) {
  return a_table_bytes(E, scalar_a) + (size_t)E * 64 * 8 + (with_u ? u_bytes(E, k, waves) : 0) +
         ring_bytes(k) * waves;
}

// One token for one lane: every slot j advances with expert e[j]'s parameters;
// returns sum_j gw[j] (C_t . h_j + Dskip[e_j] x).
//   TRACK: also decay the carried parts g (fix-up pass; with SA, g[j][0] is
//          slot j's common decay factor and g[j][1] holds max |h_in|).
//   ACC_U: accumulate Delta log2(e) per (slot, expert) (chunk pass).
//   MEM:   rows from memory at channel dd (p), sums of the exponents in lg
//          instead of U.
template <int K, bool TRACK, bool ACC_U, bool SA, bool ZOH, bool MEM = false>
__device__ __forceinline__ float slot_token(const Smem& s, float* U, int E, const int* e,
                                            const float* gw, int slot, int i, int lane, float xv,
                                            float rv, float (*h)[kN], float (*g)[kN],
                                            const SlotParams* p = nullptr, int dd = 0,
                                            float (*lg)[kN] = nullptr) {
  const float4* bc = reinterpret_cast<const float4*>(s.ring.bc + (slot * kTB + i) * 32);
  float bv[kN], cv[kN];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 b4 = bc[q], c4 = bc[4 + q];
    bv[4 * q + 0] = b4.x;
    bv[4 * q + 1] = b4.y;
    bv[4 * q + 2] = b4.z;
    bv[4 * q + 3] = b4.w;
    cv[4 * q + 0] = c4.x;
    cv[4 * q + 1] = c4.y;
    cv[4 * q + 2] = c4.z;
    cv[4 * q + 3] = c4.w;
  }
  // the token's table reads first; the U sums are written back last, so that
  // no LDS write orders the A-row reads behind the softplus chain
  float2 bdv[K];
  float uo[K], du[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if constexpr (MEM) {
      const size_t o = (size_t)e[j] * p->D + dd;
      bdv[j] = make_float2(p->bias[o], p->Dsk[o]);
    } else {
      bdv[j] = s.BD[e[j] * 64 + lane];
      if (ACC_U) uo[j] = U[(j * E + e[j]) * 64 + lane];
    }
  }
  float y = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float2 bd = bdv[j];
    const float dlt = softplus_f32(rv + bd.x);
    const float dl2 = dlt * kLog2e;
    du[j] = dl2;
    const float dx = dlt * xv;
    float yj = 0.f;
    if constexpr (SA) {
      const float av = MEM ? p->A[(size_t)e[j] * p->D + dd]
                           : reinterpret_cast<const float*>(s.A)[e[j] * 64 + lane];
      const float m = dl2 * av;
      if (MEM && ACC_U) lg[j][0] += m;
      const float a = hw_exp2(m);
      const float dxz = ZOH ? dx * zoh_phi(a, m) : dx;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        h[j][n] = fmaf(a, h[j][n], dxz * bv[n]);
        yj = fmaf(cv[n], h[j][n], yj);
      }
      if (TRACK) g[j][0] *= a;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a4 =
            MEM ? reinterpret_cast<const float4*>(p->A + ((size_t)e[j] * p->D + dd) * kN)[q]
                : s.A[(e[j] * 4 + q) * 64 + lane];
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 4 * q + r;
          const float m = dl2 * av[r];
          if (MEM && ACC_U) lg[j][n] += m;
          const float a = hw_exp2(m);
          const float inj = ZOH ? (dx * bv[n]) * zoh_phi(a, m) : dx * bv[n];
          h[j][n] = fmaf(a, h[j][n], inj);
          yj = fmaf(cv[n], h[j][n], yj);
          if (TRACK) g[j][n] *= a;
        }
      }
    }
    y = fmaf(gw[j], fmaf(bd.y, xv, yj), y);
  }
  // each lane owns its column of U, and (slot, expert) rows differ between
  // slots, so a plain read-modify-write accumulates correctly
  if (ACC_U && !MEM)
#pragma unroll
    for (int j = 0; j < K; ++j) U[(j * E + e[j]) * 64 + lane] = uo[j] + du[j];
  return y;
}

// Walk tokens [t0, t1) of sequence b for one lane, staging each block of kTB
// tokens one block ahead (as the mixed scan's walk).  With TRACK and
// `truncate`, stops once every slot's carried part has decayed on every lane.
template <typename TIn, typename TOut, int K, bool TRACK, bool ACC_U, bool SA, bool ZOH,
          bool MEM>
__device__ __forceinline__ void walk(const SlotParams& p, const Smem& s, float* U, int b, int t0,
                                     int t1, int d, bool active, int lane, bool truncate,
                                     float (*h)[kN], float (*g)[kN], float (*lg)[kN]) {
  const int dd = active ? d : p.D - 1;  // MEM: a valid channel for idle lanes
  constexpr int KW = (kTB * K + 63) / 64;
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
  int gate_bad = 0;  // the gates do not enter the states: not used
  auto valid_at = [&](int t) { return (int)min((size_t)kTB, total - (row + t)); };
  auto load_xr = [&](int t, TIn* xs, TIn* rs) {
    const int v = valid_at(t);
    const stage::rsrc_t rx = stage::rows_rsrc<TIn>(p.x, row + t, v, D);
    const stage::rsrc_t rr = stage::rows_rsrc<TIn>(p.dt, row + t, v, D);
    // the scalar offset is not range-checked: rows past the tensor's end
    // re-read its last row
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
      const uint32_t so = (uint32_t)min(i, v - 1) * xrow;
      xs[i] = stage::buf_load<TIn>(rx, xoff, so);
      rs[i] = stage::buf_load<TIn>(rr, xoff, so);
    }
  };

  st.issue(p, row + t0, valid_at(t0), K);
  load_xr(t0, xc, rc);
  st.commit(s.ring, 0, min(kTB, t1 - t0), K, p.E, lane, gate_bad);

  int slot = 0;
  for (int tb = t0; tb < t1; tb += kTB, slot ^= 1) {
    const int n = min(kTB, t1 - tb);
    const int tn = tb + kTB;
    const bool more = tn < t1;
    if (more) {
      st.issue(p, row + tn, valid_at(tn), K);
      load_xr(tn, xn, rn);
    }
    wave_sync();
    const stage::rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, n, D);
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
        const float yv = slot_token<K, TRACK, ACC_U, SA, ZOH, MEM>(
            s, U, p.E, ev, gv, slot, i, lane, to_f32(xc[i]), to_f32(rc[i]), h, g, &p, dd, lg);
        if (active) stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
      }
    }
    if (TRACK && truncate) {
      bool conv = true;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float mh = 0.f;
#pragma unroll
        for (int q = 0; q < kN; ++q) mh = fmaxf(mh, fabsf(h[j][q]));
        const float thr = fmaxf(kFixupTol * mh, kTiny);
        if constexpr (SA) {
          conv &= fabsf(g[j][0]) * g[j][1] <= thr;  // NaN: not converged
        } else {
#pragma unroll
          for (int q = 0; q < kN; ++q) conv &= fabsf(g[j][q]) <= thr;
        }
      }
      if (__all(conv)) break;
    }
    if (more) {
      st.commit(s.ring, slot ^ 1, min(kTB, t1 - tn), K, p.E, lane, gate_bad);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        xc[i] = xn[i];
        rc[i] = rn[i];
      }
    }
  }
}

// Pass 1 (or the only pass when CHUNKED is false).
template <typename TIn, typename TOut, int WAVES, int K, bool CHUNKED, bool SA, bool ZOH,
          bool MEM>
__global__ __launch_bounds__(WAVES * 64) void slot_chunk_kernel(SlotParams p) {
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const Smem s = smem_layout(MEM ? 0 : p.E, K, CHUNKED && !MEM, WAVES, wave, SA);
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  int bad = 0;
  float* U = nullptr;
  if constexpr (!MEM) {
    bad = stage::load_table(p, s.A, s.BD, d0, SA);
    U = s.U + (size_t)wave * K * p.E * 64;
    if (CHUNKED)
      for (int q = 0; q < K * p.E; ++q) U[q * 64 + lane] = 0.f;
    bad = __syncthreads_or(bad);
  } else if (CHUNKED) {
    bad = p.tflags[tile];
  }

  const int c = cg * WAVES + wave;
  if (c >= p.nchunks) return;  // no barrier below
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);

  float h[K][kN];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int n = 0; n < kN; ++n)
      h[j][n] = (c == 0 && p.h0 != nullptr && active)
                    ? p.h0[(((size_t)b * K + j) * p.D + d) * kN + n]
                    : 0.f;

  // MEM: each slot's exponent sums over the chunk (the table path keeps
  // per-expert sums U in LDS instead)
  float lg[K][kN];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int n = 0; n < kN; ++n) lg[j][n] = 0.f;
  walk<TIn, TOut, K, false, CHUNKED, SA, ZOH, MEM>(p, s, U, b, t0, t1, d, active, lane, false, h,
                                                   nullptr, lg);

  if (CHUNKED) {
    const size_t rows = (size_t)K * kN;
    const size_t base = ((size_t)b * p.nchunks + c) * rows * p.D + d;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      // slot j's total decay over the chunk: exp2(sum_e U_je A[e, d, n] log2 e)
      float m[kN];
#pragma unroll
      for (int n = 0; n < kN; ++n) m[n] = MEM ? lg[j][n] : 0.f;
      for (int e = 0; e < (MEM ? 0 : p.E); ++e) {
        const float u = U[(j * p.E + e) * 64 + lane];
        if (SA) {
          m[0] = fmaf(u, reinterpret_cast<const float*>(s.A)[e * 64 + lane], m[0]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a = s.A[(e * 4 + q) * 64 + lane];
            m[4 * q + 0] = fmaf(u, a.x, m[4 * q + 0]);
            m[4 * q + 1] = fmaf(u, a.y, m[4 * q + 1]);
            m[4 * q + 2] = fmaf(u, a.z, m[4 * q + 2]);
            m[4 * q + 3] = fmaf(u, a.w, m[4 * q + 3]);
          }
        }
      }
      if (active) {
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          const size_t r = base + (size_t)(j * kN + n) * p.D;
          p.P[r] = hw_exp2(m[SA ? 0 : n]);
          p.H[r] = h[j][n];
        }
      }
    }
    if (lane == 0) p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] = bad ? 1 : 0;
  } else if (p.h_final != nullptr && active) {
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int n = 0; n < kN; ++n)
        p.h_final[(((size_t)b * K + j) * p.D + d) * kN + n] = h[j][n];
  }
}

// Pass 3: chunks 1.. re-run from their carried-in states until every slot's
// carried part has decayed away (or to the chunk's end).
template <typename TIn, typename TOut, int WAVES, int K, bool SA, bool ZOH, bool MEM>
__global__ __launch_bounds__(WAVES * 64) void slot_fixup_kernel(SlotParams p) {
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const Smem s = smem_layout(MEM ? 0 : p.E, K, false, WAVES, wave, SA);
  const int nfix = p.nchunks - 1;
  const int ncg = (nfix + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  if constexpr (!MEM) {
    stage::load_table(p, s.A, s.BD, d0, SA);
    __syncthreads();
  }

  const int c = 1 + cg * WAVES + wave;
  if (c >= p.nchunks) return;
  const int t0 = c * p.chunk;
  const int t1 = min(p.L, t0 + p.chunk);
  const size_t base = ((size_t)b * p.nchunks + c) * (size_t)K * kN * p.D + (active ? d : 0);
  float h[K][kN], g[K][kN];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float mh = 0.f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      h[j][n] = active ? p.H[base + (size_t)(j * kN + n) * p.D] : 0.f;
      g[j][n] = h[j][n];
      mh = fmaxf(mh, fabsf(h[j][n]));
    }
    if (SA) {
      // the carried part is G * h_in: track G and max |h_in|
      g[j][0] = 1.f;
      g[j][1] = mh;
    }
  }
  const bool truncate = p.carry == SWIMBA_CARRY_FIXUP &&
                        p.flags[((size_t)b * p.nchunks + c) * p.ntiles + tile] == 0;
  walk<TIn, TOut, K, true, false, SA, ZOH, MEM>(p, s, nullptr, b, t0, t1, d, active, lane,
                                                truncate, h, g, nullptr);
}

template <typename TIn, typename TOut, int K, bool SA, bool ZOH, bool MEM>
int launch_slots_t(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  constexpr int WAVES = 4;
  SlotParams p;
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

  const size_t smem1 = MEM ? smem_bytes(0, K, false, WAVES, SA) : smem_bytes(p.E, K, true, WAVES, SA);
  const size_t smem3 = smem_bytes(MEM ? 0 : p.E, K, false, WAVES, SA);
  p.tflags = nullptr;
  if (MEM && pl.nchunks > 1) {
    // contraction check of every tile's A (the table path checks while staging)
    int32_t* tf = reinterpret_cast<int32_t*>(w + pl.off_tflags);
    p.tflags = tf;
    const int rc = launch_a_flags(p.A, p.E, p.D, SA, tf, st);
    if (rc != SWIMBA_OK) return rc;
  }
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  if (pl.nchunks <= 1) {
    p.nchunks = 1;
    const dim3 grid((unsigned)((size_t)p.B * p.ntiles));
    allow_dynamic_lds(slot_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH, MEM>, smem3);
    const int rc = launch_timed(slot_chunk_kernel<TIn, TOut, WAVES, K, false, SA, ZOH, MEM>, grid,
                                dim3(WAVES * 64), smem3, st, ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  const int ncg = (p.nchunks + WAVES - 1) / WAVES;
  const dim3 grid1((unsigned)((size_t)p.B * ncg * p.ntiles));
  allow_dynamic_lds(slot_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH, MEM>, smem1);
  int rc = launch_timed(slot_chunk_kernel<TIn, TOut, WAVES, K, true, SA, ZOH, MEM>, grid1,
                        dim3(WAVES * 64), smem1, st, ev, p);
  if (rc != SWIMBA_OK) return rc;
  // the carry pass treats the k slots as k trajectories of 16 state rows
  rc = launch_carry(p.B, p.nchunks, p.D, K, p.P, p.H, p.h_final, 1, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  const int ncg3 = (p.nchunks - 1 + WAVES - 1) / WAVES;
  const dim3 grid3((unsigned)((size_t)p.B * ncg3 * p.ntiles));
  allow_dynamic_lds(slot_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH, MEM>, smem3);
  return launch_timed(slot_fixup_kernel<TIn, TOut, WAVES, K, SA, ZOH, MEM>, grid3, dim3(WAVES * 64),
                      smem3, st, ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut, bool SA, bool ZOH>
int launch_slots_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->E > 16) {
    // rows from memory: k <= 2 (the slots' states and exponent sums in VGPRs)
    if (a->k == 1) return launch_slots_t<TIn, TOut, 1, SA, ZOH, true>(a, pl, ws, st);
    if (a->k == 2) return launch_slots_t<TIn, TOut, 2, SA, ZOH, true>(a, pl, ws, st);
    return SWIMBA_EUNSUPPORTED;
  }
  switch (a->k) {
    case 1:
      return launch_slots_t<TIn, TOut, 1, SA, ZOH, false>(a, pl, ws, st);
    case 2:
      return launch_slots_t<TIn, TOut, 2, SA, ZOH, false>(a, pl, ws, st);
    case 3:
      return launch_slots_t<TIn, TOut, 3, SA, ZOH, false>(a, pl, ws, st);
    case 4:
      return launch_slots_t<TIn, TOut, 4, SA, ZOH, false>(a, pl, ws, st);
    default:
      return SWIMBA_EUNSUPPORTED;
  }
}

template <typename TIn, typename TOut>
int launch_slots_e(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  const bool zoh = a->disc == SWIMBA_DISC_ZOH;
  if (a->a_form == SWIMBA_A_SCALAR)
    return zoh ? launch_slots_k<TIn, TOut, true, true>(a, pl, ws, st)
               : launch_slots_k<TIn, TOut, true, false>(a, pl, ws, st);
  return zoh ? launch_slots_k<TIn, TOut, false, true>(a, pl, ws, st)
             : launch_slots_k<TIn, TOut, false, false>(a, pl, ws, st);
}

}  // namespace slots
}  // namespace swimba
