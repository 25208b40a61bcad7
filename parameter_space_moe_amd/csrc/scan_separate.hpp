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
// indexing, no scratch).  Chunks are joined exactly: pass 1 runs every chunk
// from zero (chunk 0 from h0) and records each expert's end state and decay
// P_e[n] = exp2(S_e A[e,n] log2 e) with S_e the Delta summed over the tokens
// that selected e; pass 2 carries the states across chunks (shared with the
// mixed scan); pass 3 re-runs chunks 1.. from their carried-in states.
#pragma once
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

template <typename TIn, bool READOUT>
__device__ __forceinline__ float expert_update(float* h, float& S, const float4* sA,
                                               float2 bd, int lane, float xv, float rv,
                                               const TIn* Bp, const TIn* Cp) {
  const float dlt = softplus_f32(rv + bd.x);
  S += dlt;
  const float dl2 = dlt * kLog2e, dx = dlt * xv;
  float ye = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a4 = sA[q * 64 + lane];
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 4 * q + i;
      const float a = hw_exp2(dl2 * av[i]);
      h[n] = fmaf(a, h[n], dx * to_f32(Bp[n]));
      if (READOUT) ye = fmaf(to_f32(Cp[n]), h[n], ye);
    }
  }
  return READOUT ? fmaf(bd.y, xv, ye) : 0.f;
}

// Uniform dispatch to the expert `e` (compile-time register indices).
template <typename TIn, bool READOUT, int EMAX, int EE = 0>
__device__ __forceinline__ float dispatch_update(float (&H)[EMAX][kN], float (&S)[EMAX], int e,
                                                 const float4* sA, float2 bd, int lane,
                                                 float xv, float rv, const TIn* Bp,
                                                 const TIn* Cp) {
  if constexpr (EE < EMAX) {
    if (e == EE)
      return expert_update<TIn, READOUT>(H[EE], S[EE], sA + EE * 4 * 64, bd, lane, xv, rv, Bp,
                                         Cp);
    return dispatch_update<TIn, READOUT, EMAX, EE + 1>(H, S, e, sA, bd, lane, xv, rv, Bp, Cp);
  } else {
    return 0.f;
  }
}

template <typename TIn, typename TOut, int EMAX, int WAVES, int PASS>
__global__ __launch_bounds__(WAVES * 64) void sep_kernel(SepParams p) {
  extern __shared__ float4 smem_raw[];
  float4* sA = smem_raw;                                       // [E][4][64]
  float2* sBD = reinterpret_cast<float2*>(sA + p.E * 4 * 64);  // [E][64]
  const int first_chunk = PASS == kPassFixup ? 1 : 0;
  const int nwork = PASS == kPassSingle ? 1 : p.nchunks - first_chunk;
  const int ncg = (nwork + WAVES - 1) / WAVES;
  int bid = blockIdx.x;
  const int tile = bid % p.ntiles;
  bid /= p.ntiles;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int d0 = tile * 64, d = d0 + lane;
  const bool active = d < p.D;

  for (int i = threadIdx.x; i < p.E * 256; i += blockDim.x) {
    int e = i >> 8, r = i & 255, dl = r >> 2, q = r & 3, dd = d0 + dl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (dd < p.D) {
      const float* a = p.A + ((size_t)e * p.D + dd) * kN + q * 4;
      v = make_float4(a[0], a[1], a[2], a[3]);
    }
    sA[(e * 4 + q) * 64 + dl] = v;
  }
  for (int i = threadIdx.x; i < p.E * 64; i += blockDim.x) {
    int e = i >> 6, dl = i & 63, dd = d0 + dl;
    sBD[i] = dd < p.D ? make_float2(p.bias[(size_t)e * p.D + dd], p.Dsk[(size_t)e * p.D + dd])
                      : make_float2(0.f, 0.f);
  }
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

  constexpr bool kReadout = true;
  const bool write_y = PASS != kPassFirst || c == 0;
  const TIn* X = reinterpret_cast<const TIn*>(p.x);
  const TIn* R = reinterpret_cast<const TIn*>(p.dt);
  TOut* Y = reinterpret_cast<TOut*>(p.y);
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
    const TIn* Bp = reinterpret_cast<const TIn*>(p.Bm) + bt * kN;
    const TIn* Cp = reinterpret_cast<const TIn*>(p.Cm) + bt * kN;
    float yv = 0.f;
    for (int j = 0; j < p.k; ++j) {
      int e = p.idx[bt * p.k + j];
      e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
      const float gj = p.gate[bt * p.k + j];
      const float2 bd = sBD[e * 64 + lane];
      float ye;
      if (write_y)
        ye = dispatch_update<TIn, kReadout, EMAX>(H, S, e, sA, bd, lane, xv, rv, Bp, Cp);
      else
        ye = dispatch_update<TIn, false, EMAX>(H, S, e, sA, bd, lane, xv, rv, Bp, Cp);
      yv = fmaf(gj, ye, yv);
    }
    if (write_y && active) Y[off] = from_f32<TOut>(yv);
  }

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

template <typename TIn, typename TOut, int EMAX>
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
  const size_t smem = (size_t)p.E * (4 * 64 * 16 + 64 * 8);
  hipEvent_t* ev = a->phase_events;
  if (ev) (void)hipEventRecord(ev[0], st);
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassSingle>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassFirst>, smem);
  allow_dynamic_lds(sep_kernel<TIn, TOut, EMAX, W, kPassFixup>, smem);
  if (pl.nchunks <= 1) {
    hipLaunchKernelGGL((sep_kernel<TIn, TOut, EMAX, W, kPassSingle>),
                       dim3((unsigned)((size_t)p.B * p.ntiles)), dim3(W * 64), smem, st, p);
    if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
    if (ev)
      for (int i = 1; i < 4; ++i) (void)hipEventRecord(ev[i], st);
    return SWIMBA_OK;
  }
  const int ncg1 = (p.nchunks + W - 1) / W;
  hipLaunchKernelGGL((sep_kernel<TIn, TOut, EMAX, W, kPassFirst>),
                     dim3((unsigned)((size_t)p.B * ncg1 * p.ntiles)), dim3(W * 64), smem, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  if (ev) (void)hipEventRecord(ev[1], st);
  int rc = launch_carry(p.B, p.nchunks, p.D, p.E, p.P, p.H, p.h_final, 1, st);
  if (rc != SWIMBA_OK) return rc;
  if (ev) (void)hipEventRecord(ev[2], st);
  const int ncg3 = (p.nchunks - 1 + W - 1) / W;
  hipLaunchKernelGGL((sep_kernel<TIn, TOut, EMAX, W, kPassFixup>),
                     dim3((unsigned)((size_t)p.B * ncg3 * p.ntiles)), dim3(W * 64), smem, st, p);
  if (hipGetLastError() != hipSuccess) return SWIMBA_EHIP;
  if (ev) (void)hipEventRecord(ev[3], st);
  return SWIMBA_OK;
}

template <typename TIn, typename TOut>
int launch_sep_e(const swimba_scan_args* a, const ScanPlan& pl, void* ws, hipStream_t st) {
  if (a->E <= 4) return launch_sep_t<TIn, TOut, 4>(a, pl, ws, st);
  if (a->E <= 8) return launch_sep_t<TIn, TOut, 8>(a, pl, ws, st);
  return launch_sep_t<TIn, TOut, 16>(a, pl, ws, st);
}

}  // namespace sep
}  // namespace swimba
