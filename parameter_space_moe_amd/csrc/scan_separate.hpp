// Separate design ("MoE of separate SSMs") for gfx950: one state trajectory per
// expert, advanced only when the router selects that expert; the token's output
// mixes the selected experts' outputs with the gates.  Pages: "Swimba: Switch
// Mamba Model Scales State Space Models" (Spanish "Distinción de Diseños",
// French "Distinction des deux designs"; Theorem 4: the designs differ once
// routing varies over time) -- kept for the cost comparison with the mixed scan.
//
// Layout of the work.  A workgroup owns one (sequence, 64-channel tile, chunk)
// and has one wave per expert: wave e keeps expert e's 16 states, its A row
// (pre-scaled by log2 e), dt_bias and Dskip of its lane's channel in VGPRs, so
// an update needs no table lookups and no dispatch.  The workgroup stages a
// round of tokens in LDS (B_t and C_t as fp32, the routing, the tile's x and
// dt_raw); each wave walks the round and advances its state at the tokens that
// selected its expert, writing the gate-weighted output of every (token, slot)
// it owns into an LDS buffer; after a barrier the workgroup adds each token's
// k slot outputs in slot order and stores y.  Each selection is done once, so
// the work is k updates per token.
//
// ALL (the third reading of separate trajectories): every expert's wave
// advances its state at every token, whether or not the token selected the
// expert, and writes the gate-weighted output only to the slots that chose it;
// that is E updates per token.
//
// Chunks are joined exactly: pass 1 runs every chunk from zero (chunk 0 from
// h0) and records each expert's end state and decay P_e[n] = exp2(S_e A'[e,n]),
// with S_e the Delta summed over the chunk's selections of e (ALL: over all
// its tokens) and A' = A log2 e;
// pass 2 carries the states across chunks (shared with the mixed scan); pass 3
// re-runs chunks 1.. from their carried-in states.
#pragma once
#include "scan_common.hpp"
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace sep {

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

// Tokens staged per round; the per-slot output buffer [round][k][64] bounds it.
__host__ __device__ constexpr int round_tokens(int k) {
  return k <= 2 ? 64 : (k <= 4 ? 32 : (k <= 8 ? 16 : 8));
}

template <typename TIn>
__host__ __device__ constexpr size_t sep_smem_bytes(int k) {
  return (size_t)round_tokens(k) *
         (32 * 4 + (size_t)k * 64 * 4 + 2 * (size_t)k * 4 + 2 * 64 * sizeof(TIn));
}

template <typename TIn>
struct SepSmem {
  float* bc;    // [R][32]     B_t then C_t, fp32
  float* yb;    // [R][k][64]  gate-weighted output of each (token, slot)
  int32_t* e;   // [R][k]      selected experts
  float* g;     // [R][k]      gates
  TIn* xs;      // [R][64]     x of the tile
  TIn* rs;      // [R][64]     dt_raw of the tile
};

template <typename TIn>
__device__ __forceinline__ SepSmem<TIn> sep_layout(int k) {
  extern __shared__ float4 smem_raw[];
  const int R = round_tokens(k);
  char* p = reinterpret_cast<char*>(smem_raw);
  SepSmem<TIn> s;
  s.bc = reinterpret_cast<float*>(p);
  p += (size_t)R * 32 * 4;
  s.yb = reinterpret_cast<float*>(p);
  p += (size_t)R * k * 64 * 4;
  s.e = reinterpret_cast<int32_t*>(p);
  p += (size_t)R * k * 4;
  s.g = reinterpret_cast<float*>(p);
  p += (size_t)R * k * 4;
  s.xs = reinterpret_cast<TIn*>(p);
  p += (size_t)R * 64 * sizeof(TIn);
  s.rs = reinterpret_cast<TIn*>(p);
  return s;
}

// Stage tokens [ts, ts + n) of sequence row `row` for the tile at d0 (all
// threads of the workgroup).
template <typename TIn>
__device__ __forceinline__ void stage_round(const SepParams& p, const SepSmem<TIn>& s,
                                            size_t row, int ts, int n, int k, int d0) {
  const int nthr = blockDim.x, tid = threadIdx.x;
  const TIn* Bm = reinterpret_cast<const TIn*>(p.Bm) + (row + ts) * kN;
  const TIn* Cm = reinterpret_cast<const TIn*>(p.Cm) + (row + ts) * kN;
  for (int q = tid; q < 2 * n * kN; q += nthr) {
    const int which = q >= n * kN, r = which ? q - n * kN : q;
    const float v = to_f32(which ? Cm[r] : Bm[r]);
    s.bc[(r / kN) * 32 + which * kN + (r % kN)] = v;
  }
  const int32_t* ib = p.idx + (row + ts) * k;
  const float* gb = p.gate + (row + ts) * k;
  for (int q = tid; q < n * k; q += nthr) {
    int e = ib[q];
    s.e[q] = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
    s.g[q] = gb[q];
  }
  const TIn* X = reinterpret_cast<const TIn*>(p.x) + (row + ts) * p.D + d0;
  const TIn* Rr = reinterpret_cast<const TIn*>(p.dt) + (row + ts) * p.D + d0;
  const int width = min(64, p.D - d0);
  for (int q = tid; q < n * 64; q += nthr) {
    const int i = q >> 6, c = q & 63;
    const bool ok = c < width;
    const size_t o = (size_t)i * p.D + (ok ? c : 0);
    const TIn xv = X[o], rv = Rr[o];
    s.xs[q] = ok ? xv : TIn(0);
    s.rs[q] = ok ? rv : TIn(0);
  }
}

// Advance this wave's expert by one selected token; returns the expert's
// output C_t . h + Dskip x (READOUT) or 0.  SA: one transition Ae[0] shared
// by the 16 states.  ZOH: zero-order-hold input term (zoh_phi times Euler).
template <bool READOUT, bool SA, bool ZOH>
__device__ __forceinline__ float expert_step(float* h, float& S, const float* Ae, float bias,
                                             float dsk, float xv, float rv, const float4* bc) {
  const float dlt = softplus_f32(rv + bias);
  S += dlt;
  const float dx = dlt * xv;
  const float a0 = SA ? hw_exp2(dlt * Ae[0]) : 0.f;
  const float dx0 = (SA && ZOH) ? dx * zoh_phi(a0, dlt * Ae[0]) : dx;
  float ye = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 b4 = bc[q], c4 = bc[4 + q];
    const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * q + r;
      const float a = SA ? a0 : hw_exp2(dlt * Ae[n]);
      const float inj = (ZOH && !SA) ? (dx * bv[r]) * zoh_phi(a, dlt * Ae[n]) : dx0 * bv[r];
      h[n] = fmaf(a, h[n], inj);
      if (READOUT) ye = fmaf(cv[r], h[n], ye);
    }
  }
  return READOUT ? fmaf(dsk, xv, ye) : 0.f;
}

// One round: this wave's selections among tokens [0, n) of the staged round,
// in token order and, within a token, in slot order.  With k known at compile
// time the wave first takes one ballot per slot (which staged tokens chose its
// expert there) and then visits only the selected tokens, so the scan over
// the round costs scalar bit operations only.
template <typename TIn, int K, bool READOUT, bool SA, bool ZOH, bool ALL>
__device__ __forceinline__ void walk_round(const SepSmem<TIn>& s, int n, int k, int ex, int lane,
                                           float* h, float& S, const float* Ae, float bias,
                                           float dsk) {
  if constexpr (ALL) {
    // every token advances the state; the output goes to the slots that
    // selected this expert (none, one, or several)
    for (int i = 0; i < n; ++i) {
      const float xv = to_f32(s.xs[i * 64 + lane]), rv = to_f32(s.rs[i * 64 + lane]);
      const float4* bc = reinterpret_cast<const float4*>(s.bc + i * 32);
      const float ye = expert_step<READOUT, SA, ZOH>(h, S, Ae, bias, dsk, xv, rv, bc);
      if (READOUT) {
#pragma unroll
        for (int j = 0; j < (K > 0 ? K : 16); ++j) {
          if (K == 0 && j >= k) break;
          if (uniform(s.e[i * k + j]) == ex) s.yb[(i * k + j) * 64 + lane] = s.g[i * k + j] * ye;
        }
      }
    }
    return;
  }
  auto select = [&](int i, int j) {
    const float xv = to_f32(s.xs[i * 64 + lane]), rv = to_f32(s.rs[i * 64 + lane]);
    const float4* bc = reinterpret_cast<const float4*>(s.bc + i * 32);
    const float ye = expert_step<READOUT, SA, ZOH>(h, S, Ae, bias, dsk, xv, rv, bc);
    if (READOUT) s.yb[(i * k + j) * 64 + lane] = s.g[i * k + j] * ye;
  };
  if constexpr (K > 0) {
    uint64_t m[K], any = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool sel = lane < n && s.e[(lane < n ? lane : 0) * K + j] == ex;
      m[j] = __ballot(sel);
      any |= m[j];
    }
    while (any != 0) {
      const int i = __builtin_ctzll(any);
      any &= any - 1;
#pragma unroll
      for (int j = 0; j < K; ++j)
        if ((m[j] >> i) & 1) select(i, j);
    }
  } else {
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < k; ++j)
        if (uniform(s.e[i * k + j]) == ex) select(i, j);
  }
}

template <typename TIn, typename TOut, int PASS, int K, bool SA, bool ZOH, bool ALL>
__global__ __launch_bounds__(1024) void sep_kernel(SepParams p) {
  const int k = K > 0 ? K : p.k;
  const int R = round_tokens(k);
  const int tid = threadIdx.x, lane = tid & 63, nthr = blockDim.x;
  const int ex = uniform((int)(threadIdx.x >> 6));  // this wave's expert
  const SepSmem<TIn> s = sep_layout<TIn>(k);

  const int first = PASS == kPassFixup ? 1 : 0;
  const int nwork = PASS == kPassSingle ? 1 : p.nchunks - first;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int c = first + bid % nwork;
  const int b = bid / nwork;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;
  const int dd = active ? d : p.D - 1;
  const int chunk = PASS == kPassSingle ? p.L : p.chunk;
  const int t0 = c * chunk, t1 = min(p.L, t0 + chunk);
  const size_t row = (size_t)b * p.L;
  const int rows = p.E * kN;

  float Ae[kN], h[kN];
  if (SA) {
    Ae[0] = p.A[(size_t)ex * p.D + dd] * kLog2e;
  } else {
    const float* Ap = p.A + ((size_t)ex * p.D + dd) * kN;
#pragma unroll
    for (int n = 0; n < kN; ++n) Ae[n] = Ap[n] * kLog2e;
  }
  const float bias = p.bias[(size_t)ex * p.D + dd], dsk = p.Dsk[(size_t)ex * p.D + dd];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    float v = 0.f;
    if (active) {
      if (PASS == kPassFixup)
        v = p.H[(((size_t)b * p.nchunks + c) * rows + ex * kN + n) * p.D + d];
      else if (c == 0 && p.h0 != nullptr)
        v = p.h0[(((size_t)b * p.E + ex) * p.D + d) * kN + n];
    }
    h[n] = v;
  }
  float S = 0.f;
  // pass 1 needs no output for chunks >= 1 (pass 3 recomputes them)
  const bool readout = PASS != kPassFirst || c == 0;
  TOut* Y = reinterpret_cast<TOut*>(p.y);

  for (int ts = t0; ts < t1; ts += R) {
    const int n = min(R, t1 - ts);
    stage_round<TIn>(p, s, row, ts, n, k, d0);
    __syncthreads();
    if (readout)
      walk_round<TIn, K, true, SA, ZOH, ALL>(s, n, k, ex, lane, h, S, Ae, bias, dsk);
    else
      walk_round<TIn, K, false, SA, ZOH, ALL>(s, n, k, ex, lane, h, S, Ae, bias, dsk);
    __syncthreads();
    // every (token, slot) output was written by its expert's wave; add them in
    // slot order.  The next round's staging touches no output buffer, and its
    // barrier comes before any wave writes the buffer again.
    if (readout) {
      for (int q = tid; q < n * 64; q += nthr) {
        const int i = q >> 6, cl = q & 63;
        if (d0 + cl < p.D) {
          float v = s.yb[(i * k) * 64 + cl];
          for (int j = 1; j < k; ++j) v += s.yb[(i * k + j) * 64 + cl];
          Y[(row + ts + i) * p.D + d0 + cl] = from_f32<TOut>(v);
        }
      }
    }
  }

  if (PASS == kPassFirst) {
    if (active) {
      const size_t base = ((size_t)b * p.nchunks + c) * rows + ex * kN;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        p.P[(base + n) * p.D + d] = hw_exp2(S * Ae[SA ? 0 : n]);
        p.H[(base + n) * p.D + d] = h[n];
      }
    }
  } else if (PASS == kPassSingle && p.h_final != nullptr && active) {
#pragma unroll
    for (int n = 0; n < kN; ++n) p.h_final[(((size_t)b * p.E + ex) * p.D + d) * kN + n] = h[n];
  }
}

template <typename TIn, typename TOut, int K, bool SA, bool ZOH, bool ALL>
int launch_sep_t(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
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
  const size_t smem = sep_smem_bytes<TIn>(p.k);
  const dim3 block((unsigned)(p.E * 64));
  const size_t tiles = (size_t)p.B * p.ntiles;
  const hipEvent_t* ev = a->phase_events;  // (start, end) x (chunk, carry, fix-up)
  allow_dynamic_lds(sep_kernel<TIn, TOut, kPassSingle, K, SA, ZOH, ALL>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, kPassFirst, K, SA, ZOH, ALL>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, kPassFixup, K, SA, ZOH, ALL>, smem);
  if (pl.nchunks <= 1) {
    const int rc = launch_timed(sep_kernel<TIn, TOut, kPassSingle, K, SA, ZOH, ALL>, dim3((unsigned)tiles),
                                block, smem, st, ev, p);
    if (rc != SWIMBA_OK) return rc;
    record_skipped(ev ? ev + 2 : nullptr, st);
    record_skipped(ev ? ev + 4 : nullptr, st);
    return SWIMBA_OK;
  }
  int rc = launch_timed(sep_kernel<TIn, TOut, kPassFirst, K, SA, ZOH, ALL>,
                        dim3((unsigned)(tiles * p.nchunks)), block, smem, st, ev, p);
  if (rc != SWIMBA_OK) return rc;
  rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 1, st, ev ? ev + 2 : nullptr);
  if (rc != SWIMBA_OK) return rc;
  return launch_timed(sep_kernel<TIn, TOut, kPassFixup, K, SA, ZOH, ALL>,
                      dim3((unsigned)(tiles * (p.nchunks - 1))), block, smem, st,
                      ev ? ev + 4 : nullptr, p);
}

template <typename TIn, typename TOut, bool SA, bool ZOH, bool ALL>
int launch_sep_k(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  switch (a->k) {
    case 1:
      return launch_sep_t<TIn, TOut, 1, SA, ZOH, ALL>(a, pl, ws, st);
    case 2:
      return launch_sep_t<TIn, TOut, 2, SA, ZOH, ALL>(a, pl, ws, st);
    default:
      return launch_sep_t<TIn, TOut, 0, SA, ZOH, ALL>(a, pl, ws, st);
  }
}

template <typename TIn, typename TOut, bool ALL>
int launch_sep_z(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  const bool zoh = a->disc == SWIMBA_DISC_ZOH;
  if (a->a_form == SWIMBA_A_SCALAR)
    return zoh ? launch_sep_k<TIn, TOut, true, true, ALL>(a, pl, ws, st)
               : launch_sep_k<TIn, TOut, true, false, ALL>(a, pl, ws, st);
  return zoh ? launch_sep_k<TIn, TOut, false, true, ALL>(a, pl, ws, st)
             : launch_sep_k<TIn, TOut, false, false, ALL>(a, pl, ws, st);
}

// all: every expert advances at every token (the all-experts reading)
template <typename TIn, typename TOut>
int launch_sep_e(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st,
                 bool all) {
  return all ? launch_sep_z<TIn, TOut, true>(a, pl, ws, st)
             : launch_sep_z<TIn, TOut, false>(a, pl, ws, st);
}

}  // namespace sep
}  // namespace swimba
