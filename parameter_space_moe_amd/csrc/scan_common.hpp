// Shared staging pieces of the chunked scans (mixed and separate designs):
// the per-wave LDS ring of wave-uniform per-token data, its vector-load
// staging one block ahead, and the expert table of a 64-channel tile.
//
// Parameter structs used with these templates provide: int L, E; const void
// *Bm, *Cm; const int32_t* idx; const float* gate, *A, *bias, *Dsk; int D.
#pragma once
#include "swimba_device.hpp"
#include "swimba_internal.hpp"

namespace swimba {
namespace stage {

constexpr int kTB = 8;  // tokens per staging block

// Per-wave LDS ring holding the wave-uniform data of two blocks of kTB tokens:
// B_t and C_t as fp32 (32 floats per token), the selected experts and gates.
struct Ring {
  float* bc;    // [2][kTB][32]
  int32_t* e;   // [2][kTB][k]
  float* g;     // [2][kTB][k]
};

__host__ __device__ constexpr size_t ring_bytes(int k) {
  return (size_t)2 * kTB * 32 * 4 + (size_t)2 * 2 * kTB * k * 4;
}

// Stage the tile's expert parameters; returns 1 if any A in the tile is not
// strictly negative (including NaN).
template <typename P>
__device__ __forceinline__ int load_table(const P& p, float4* sA, float2* sBD, int d0) {
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
    sA[(e * 4 + q) * 64 + dl] = v;
  }
  for (int i = threadIdx.x; i < p.E * 64; i += nthr) {
    int e = i >> 6, dl = i & 63, d = d0 + dl;
    float2 v = make_float2(0.f, 0.f);
    if (d < p.D) v = make_float2(p.bias[(size_t)e * p.D + d], p.Dsk[(size_t)e * p.D + d]);
    sBD[i] = v;
  }
  return bad;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Registers of one block's staging loads: a 16-byte piece of B_t or C_t per
// lane, and up to KW routing words (idx, then gates).
template <int KW>
struct StageRegs {
  uint4 piece;
  int32_t word[KW];
};

// Issue the loads of tokens [tb, tb + n) of sequence row `row` (n >= 1).  The
// loads are unconditional -- positions past the block's last token re-read
// that token -- so no branch waits on them before the commit.
template <typename TIn, int KW, typename P>
__device__ __forceinline__ void stage_issue(const P& p, size_t row, int tb, int n,
                                            int k, int lane, StageRegs<KW>& r) {
  constexpr int PPT = 16 * (int)sizeof(TIn) / 16;  // 16-byte pieces per token per vector
  constexpr int NP = 2 * kTB * PPT;
  const int q = lane < NP ? lane : NP - 1;
  const int arr = q / (kTB * PPT), rr = q % (kTB * PPT), part = rr % PPT;
  const int tok = min(rr / PPT, n - 1);
  const TIn* base = reinterpret_cast<const TIn*>(arr ? p.Cm : p.Bm) + (row + tb) * kN;
  const uint32_t o = (uint32_t)(tok * kN + part * (16 / (int)sizeof(TIn)));
  r.piece = at32(reinterpret_cast<const uint4*>(base), o / (16 / (uint32_t)sizeof(TIn)));
  const int nw = kTB * k;
  const int32_t* ib = p.idx + (row + tb) * k;
  const int32_t* gb = reinterpret_cast<const int32_t*>(p.gate) + (row + tb) * k;
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    int w = lane + 64 * i;
    w = w < 2 * nw ? w : 2 * nw - 1;
    const int arr2 = w / nw, r2 = w % nw;
    const uint32_t at = (uint32_t)(min(r2 / k, n - 1) * k + r2 % k);
    r.word[i] = arr2 ? at32(gb, at) : at32(ib, at);
  }
}

// Convert the issued loads and write them to ring slot `slot`.
template <typename TIn, int KW, typename P>
__device__ __forceinline__ void stage_commit(const P& p, const Ring& ring, int slot,
                                             int n, int k, int lane, const StageRegs<KW>& r,
                                             int& gate_bad) {
  constexpr int PPT = 16 * (int)sizeof(TIn) / 16;
  const int q = lane;
  if (q < 2 * kTB * PPT) {
    const int arr = q / (kTB * PPT), rr = q % (kTB * PPT), tok = rr / PPT, part = rr % PPT;
    float* dst = ring.bc + (slot * kTB + tok) * 32 + arr * 16 + part * (16 / sizeof(TIn));
    if (sizeof(TIn) == 2) {
      const uint32_t w4[4] = {r.piece.x, r.piece.y, r.piece.z, r.piece.w};
      float4 lo = make_float4(__uint_as_float(w4[0] << 16), __uint_as_float(w4[0] & 0xffff0000u),
                              __uint_as_float(w4[1] << 16), __uint_as_float(w4[1] & 0xffff0000u));
      float4 hi = make_float4(__uint_as_float(w4[2] << 16), __uint_as_float(w4[2] & 0xffff0000u),
                              __uint_as_float(w4[3] << 16), __uint_as_float(w4[3] & 0xffff0000u));
      reinterpret_cast<float4*>(dst)[0] = lo;
      reinterpret_cast<float4*>(dst)[1] = hi;
    } else {
      *reinterpret_cast<float4*>(dst) =
          make_float4(__uint_as_float(r.piece.x), __uint_as_float(r.piece.y),
                      __uint_as_float(r.piece.z), __uint_as_float(r.piece.w));
    }
  }
  const int nw = kTB * k;
#pragma unroll
  for (int i = 0; i < KW; ++i) {
    const int w = lane + 64 * i;
    if (w < 2 * nw) {
      const int arr = w / nw, rr = w % nw, tok = rr / k;
      if (arr == 0) {
        int e = r.word[i];
        e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
        ring.e[slot * nw + rr] = e;
      } else {
        const float gv = __int_as_float(r.word[i]);
        if (tok < n) gate_bad |= !(gv >= 0.f);
        ring.g[slot * nw + rr] = gv;
      }
    }
  }
}

}  // namespace stage
}  // namespace swimba
