// Separate design ("MoE of separate SSMs") for gfx950: one state trajectory per
// expert, advanced only when the router selects that expert; the token's output
// mixes the selected experts' outputs with the gates.  Pages: "Swimba: Switch
// Mamba Model Scales State Space Models" (Spanish "Distinción de Diseños",
// French "Distinction des deux designs"; Theorem 4: the designs differ once
// routing varies over time) -- kept for the cost comparison with the mixed scan.
//
// A lane owns one channel and holds the E x 16 expert states in VGPRs.  The
// selected expert is wave-uniform, so the update of H[e] is reached through a
// uniform branch to code with constant register indices (no dynamic VGPR
// indexing, no scratch).  Per-token routing and B_t/C_t are staged through the
// same per-wave LDS ring as the mixed scan, one block of tokens ahead.  Chunks are joined exactly: pass 1 runs every chunk
// from zero (chunk 0 from h0) and records each expert's end state and decay
// P_e[n] = exp2(S_e A[e,n] log2 e) with S_e the Delta summed over the tokens
// that selected e; pass 2 carries the states across chunks (shared with the
// mixed scan); pass 3 re-runs chunks 1.. from their carried-in states.
#pragma once
#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace sep {

using stage::kTB;
using stage::Ring;
using stage::ring_bytes;
using stage::wave_sync;

struct SepParams {
  int B, L, D, E, k;
  int chunk, nchunks, ntiles;
  const void* x;
  const void* dt;
  const void* Bm;
  const void* Cm;
  const int32_t* idx;
  const float* gate;
  const float* A;
  const float* bias;
  const float* Dsk;
  const float* h0;   // [B][E][D][16]
  void* y;
  float* h_final;    // [B][E][D][16]
  float* P;          // [B][C][E*16][D]
  float* H;          // [B][C][E*16][D]
};

enum { kPassFirst = 0, kPassFixup = 1, kPassSingle = 2 };

__host__ inline size_t sep_smem_bytes(int E, int k, int waves) {
  return (size_t)E * (4 * 64 * 16 + 64 * 8) + ring_bytes(k) * waves;
}

// Advance expert state h (16 entries) by one token with the expert's own
// parameters (its A row a4, bias/Dskip bd, already read); returns that
// expert's output (READOUT) or 0.
template <bool READOUT>
__device__ __forceinline__ float expert_update(float* h, float& S, const float4* a4, float2 bd,
                                               float xv, float rv, const float4* b4,
                                               const float4* c4) {
  const float dlt = softplus_f32(rv + bd.x);
  S += dlt;
  const float dl2 = dlt * kLog2e, dx = dlt * xv;
  float ye = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float av[4] = {a4[q].x, a4[q].y, a4[q].z, a4[q].w};
    const float bv[4] = {b4[q].x, b4[q].y, b4[q].z, b4[q].w};
    const float cv[4] = {c4[q].x, c4[q].y, c4[q].z, c4[q].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 4 * q + i;
      const float a = hw_exp2(dl2 * av[i]);
      h[n] = fmaf(a, h[n], dx * bv[i]);
      if (READOUT) ye = fmaf(cv[i], h[n], ye);
    }
  }
  return READOUT ? fmaf(bd.y, xv, ye) : 0.f;
}

// Uniform dispatch to expert `e` (compile-time register indices).
template <bool READOUT, int EMAX, int EE = 0>
__device__ __forceinline__ float dispatch_update(float (&H)[EMAX][kN], float (&S)[EMAX], int e,
                                                 const float4* a4, float2 bd, float xv, float rv,
                                                 const float4* b4, const float4* c4) {
  if constexpr (EE < EMAX) {
    if (e == EE) return expert_update<READOUT>(H[EE], S[EE], a4, bd, xv, rv, b4, c4);
    return dispatch_update<READOUT, EMAX, EE + 1>(H, S, e, a4, bd, xv, rv, b4, c4);
  } else {
    return 0.f;
  }
}

// One token for one lane: all LDS reads of the token (B_t, C_t, the selected
// experts' A rows and bias/Dskip) are issued before the uniform dispatches.
template <bool READOUT, int EMAX, int K>
__device__ __forceinline__ float sep_token(float (&H)[EMAX][kN], float (&S)[EMAX], const int* e,
                                           const float* gw, int k, const float4* sA,
                                           const float2* sBD, const float4* bc, int lane, float xv,
                                           float rv) {
  float4 b4[4], c4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    b4[q] = bc[q];
    c4[q] = bc[4 + q];
  }
  float yv = 0.f;
  auto slot = [&](int j, const float4* a4, float2 bd) {
    const float ye = dispatch_update<READOUT, EMAX>(H, S, e[j], a4, bd, xv, rv, b4, c4);
    yv = fmaf(gw[j], ye, yv);
  };
  if constexpr (K > 0) {
    float4 a4[K][4];
    float2 bd[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      bd[j] = sBD[e[j] * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[j][q] = sA[(e[j] * 4 + q) * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) slot(j, a4[j], bd[j]);
  } else {
    for (int j = 0; j < k; ++j) {
      float4 a4[4];
      const float2 bd = sBD[e[j] * 64 + lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[q] = sA[(e[j] * 4 + q) * 64 + lane];
      slot(j, a4, bd);
    }
  }
  return yv;
}

// Walk tokens [t0, t1) for one lane with the staged pipeline of the mixed
// scan.  READOUT: produce and store y.
template <typename TIn, typename TOut, int EMAX, int K, bool READOUT>
__device__ __forceinline__ void walk_sep(const SepParams& p, const float4* sA, const float2* sBD,
                                         const Ring& ring, int b, int t0, int t1, int d,
                                         bool active, int lane, float (&H)[EMAX][kN],
                                         float (&S)[EMAX]) {
  constexpr int KW = (kTB * (K > 0 ? K : 16) + 63) / 64;
  const int k = K > 0 ? K : p.k;
  const int D = p.D;
  const size_t row = (size_t)b * p.L;
  const size_t total = (size_t)p.B * p.L;
  const uint32_t xoff = (uint32_t)d * (uint32_t)sizeof(TIn);
  const uint32_t yoff = (uint32_t)d * (uint32_t)sizeof(TOut);
  const uint32_t xrow = (uint32_t)D * (uint32_t)sizeof(TIn);
  const uint32_t yrow = (uint32_t)D * (uint32_t)sizeof(TOut);
  TIn xc[kTB], rc[kTB], xn[kTB], rn[kTB];
  stage::Stager<TIn, KW> st;
  st.init(lane);
  int gate_bad = 0;
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
  st.commit(ring, 0, min(kTB, t1 - t0), k, p.E, lane, gate_bad);

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
    const stage::rsrc_t ry = stage::rows_rsrc<TOut>(p.y, row + tb, n, D);
    if constexpr (K > 0) {
      // the block's routing, once, into SGPRs
      int eb[kTB * K];
      float gb[kTB * K];
#pragma unroll
      for (int w = 0; w < kTB * K; ++w) {
        eb[w] = uniform(ring.e[slot * kTB * K + w]);
        gb[w] = uniform(ring.g[slot * kTB * K + w]);
      }
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          const float xv = active ? to_f32(xc[i]) : 0.f, rv = active ? to_f32(rc[i]) : 0.f;
          const float4* bc = reinterpret_cast<const float4*>(ring.bc + (slot * kTB + i) * 32);
          const float yv = sep_token<READOUT, EMAX, K>(H, S, eb + i * K, gb + i * K, K, sA, sBD,
                                                       bc, lane, xv, rv);
          if (READOUT && active)
            stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        if (i < n) {
          int eb[16];
          float gb[16];
          for (int j = 0; j < k; ++j) {
            eb[j] = uniform(ring.e[(slot * kTB + i) * k + j]);
            gb[j] = uniform(ring.g[(slot * kTB + i) * k + j]);
          }
          const float xv = active ? to_f32(xc[i]) : 0.f, rv = active ? to_f32(rc[i]) : 0.f;
          const float4* bc = reinterpret_cast<const float4*>(ring.bc + (slot * kTB + i) * 32);
          const float yv = sep_token<READOUT, EMAX, K>(H, S, eb, gb, k, sA, sBD, bc, lane, xv, rv);
          if (READOUT && active)
            stage::buf_store(ry, yoff, (uint32_t)i * yrow, from_f32<TOut>(yv));
        }
      }
    }
    if (more) {
      st.commit(ring, slot ^ 1, min(kTB, t1 - tn), k, p.E, lane, gate_bad);
#pragma unroll
      for (int i = 0; i < kTB; ++i) {
        xc[i] = xn[i];
        rc[i] = rn[i];
      }
    }
  }
}

template <typename TIn, typename TOut, int EMAX, int WAVES, int PASS, int K>
__global__ __launch_bounds__(WAVES * 64) void sep_kernel(SepParams p) {
  extern __shared__ float4 smem_raw[];
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int k = K > 0 ? K : p.k;
  float4* sA = smem_raw;                                       // [E][4][64]
  float2* sBD = reinterpret_cast<float2*>(sA + p.E * 4 * 64);  // [E][64]
  char* rp = reinterpret_cast<char*>(sBD + p.E * 64) + ring_bytes(k) * wave;
  Ring ring;
  ring.bc = reinterpret_cast<float*>(rp);
  ring.e = reinterpret_cast<int32_t*>(rp + 2 * kTB * 32 * 4);
  ring.g = reinterpret_cast<float*>(rp + 2 * kTB * 32 * 4 + 2 * kTB * k * 4);

  const int first_chunk = PASS == kPassFixup ? 1 : 0;
  const int nwork = PASS == kPassSingle ? 1 : p.nchunks - first_chunk;
  const int ncg = (nwork + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  stage::load_table(p, sA, sBD, d0);
  __syncthreads();

  const int c = first_chunk + cg * WAVES + wave;
  if (cg * WAVES + wave >= nwork) return;
  const int chunk = PASS == kPassSingle ? p.L : p.chunk;
  const int t0 = c * chunk;
  const int t1 = min(p.L, t0 + chunk);
  const int rows = p.E * kN;

  float H[EMAX][kN], S[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    S[e] = 0.f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      float v = 0.f;
      if (e < p.E && active) {
        if (PASS == kPassFixup)
          v = p.H[(((size_t)b * p.nchunks + c) * rows + e * kN + n) * p.D + d];
        else if (c == 0 && p.h0 != nullptr)
          v = p.h0[(((size_t)b * p.E + e) * p.D + d) * kN + n];
      }
      H[e][n] = v;
    }
  }

  // pass 1 needs no output for chunks >= 1 (pass 3 recomputes them)
  const bool readout = PASS != kPassFirst || c == 0;
  if (readout)
    walk_sep<TIn, TOut, EMAX, K, true>(p, sA, sBD, ring, b, t0, t1, d, active, lane, H, S);
  else
    walk_sep<TIn, TOut, EMAX, K, false>(p, sA, sBD, ring, b, t0, t1, d, active, lane, H, S);

  if (PASS == kPassFirst) {
    if (active) {
      const size_t base = ((size_t)b * p.nchunks + c) * rows;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e >= p.E) continue;
        const float s2 = S[e] * kLog2e;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a4 = sA[(e * 4 + q) * 64 + lane];
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = 4 * q + i;
            p.P[(base + e * kN + n) * p.D + d] = hw_exp2(s2 * av[i]);
            p.H[(base + e * kN + n) * p.D + d] = H[e][n];
          }
        }
      }
    }
  } else if (PASS == kPassSingle && p.h_final != nullptr && active) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e >= p.E) continue;
#pragma unroll
      for (int n = 0; n < kN; ++n) p.h_final[(((size_t)b * p.E + e) * p.D + d) * kN + n] = H[e][n];
    }
  }
}

template <typename TIn, typename TOut, int EMAX, int K>
int launch_sep_t(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  constexpr int W = 4;
  SepParams p;
  p.B = a->B;
  p.L = a->L;
  p.D = a->D;
  p.E = a->E;
  p.k = a->k;
  p.chunk = pl.chunk;
  p.nchunks = pl.nchunks;
  p.ntiles = pl.ntiles;
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
  const size_t smem = sep_smem_bytes(p.E, p.k, W);
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassSingle, K>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassFirst, K>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassFixup, K>, smem);
  if (pl.nchunks <= 1) {
    const int rc = launch_timed(sep_kernel<TIn, TOut, EMAX, W, kPassSingle, K>,
                                dim3((unsigned)((size_t)p.B * p.ntiles)), dim3(W * 64), smem, st,
                                ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  const int ncg1 = (p.nchunks + W - 1) / W;
  int rc = launch_timed(sep_kernel<TIn, TOut, EMAX, W, kPassFirst, K>,
                        dim3((unsigned)((size_t)p.B * ncg1 * p.ntiles)), dim3(W * 64), smem, st,
                        ev, p);
  if (rc != SWIMBA_OK) return rc;
  rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 1, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  const int ncg3 = (p.nchunks - 1 + W - 1) / W;
  return launch_timed(sep_kernel<TIn, TOut, EMAX, W, kPassFixup, K>,
                      dim3((unsigned)((size_t)p.B * ncg3 * p.ntiles)), dim3(W * 64), smem, st,
                      ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut, int EMAX>
int launch_sep_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_sep_t<TIn, TOut, EMAX, 1>(a, pl, ws, st);
    case 2:
      return launch_sep_t<TIn, TOut, EMAX, 2>(a, pl, ws, st);
    default:
      return launch_sep_t<TIn, TOut, EMAX, 0>(a, pl, ws, st);
  }
}

template <typename TIn, typename TOut>
int launch_sep_e(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->E <= 4) return launch_sep_k<TIn, TOut, 4>(a, pl, ws, st);
  if (a->E <= 8) return launch_sep_k<TIn, TOut, 8>(a, pl, ws, st);
  return launch_sep_k<TIn, TOut, 16>(a, pl, ws, st);
}

}  // namespace sep
}  // namespace swimba
